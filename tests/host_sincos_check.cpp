// Host-side driver for the library's rotary sine/cosine (csrc/rope_math.h):
// reads hexadecimal doubles from stdin, prints the sine and cosine as
// hexadecimal doubles per line.  Built with hipcc --offload-host-only by
// tests/test_kernel_helpers_host.py; nothing touches a GPU.
#include <cstdio>
#include <cstdlib>

#include "rope_math.h"

int main() {
    char buf[128];
    while (std::scanf("%127s", buf) == 1) {
        const double x = std::strtod(buf, nullptr);
        double s, c;
        kvd::rope_sincos(x, s, c);
        std::printf("%a %a\n", s, c);
    }
    return 0;
}
