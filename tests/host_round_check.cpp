// Host-side driver for the library's bf16 rounding helpers (csrc/bf16_round.h):
// reads hexadecimal doubles from stdin, prints "<bf16 from fp64> <bf16 from
// fp32 of the value>" per line.  Built with hipcc --offload-host-only by
// tests/test_kernel_helpers_host.py; nothing touches a GPU.
#include <cstdio>
#include <cstdlib>

#include "bf16_round.h"

int main() {
    char buf[128];
    while (std::scanf("%127s", buf) == 1) {
        double x = std::strtod(buf, nullptr);
        std::printf("%u %u\n", (unsigned)kvd::bf16_from_f64(x), (unsigned)kvd::bf16_from_f32((float)x));
    }
    return 0;
}
