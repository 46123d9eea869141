// Sanitizer driver for the library's host logic (test infrastructure): built
// against a host-only, AddressSanitizer + UndefinedBehaviorSanitizer build of
// the library, it calls the planners and argument checks of every entry
// point (plain, transposed B, block-scaled) on edge and random arguments —
// sizes from 0 to the largest accepted, leading dimensions at and above the
// row width, 2- and 16-byte aligned stand-in pointers, every variant and
// configuration index including out-of-range ones, forced split counts and
// workspace caps — and checks the plans' invariants. No GPU is touched:
// stand-in pointers are never dereferenced, and the library's host logic
// makes no device call. Exits 0 when every invariant holds; any
// out-of-bounds access, overflow or other undefined behaviour is reported by
// the sanitizers, which then make the process fail.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tlg.h"

static uint64_t rng_state = 0x243f6a8885a308d3ull;
static uint64_t rnd() {
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 2685821657736338717ull;
}
static int64_t pick(const int64_t *v, int n) { return v[rnd() % (uint64_t)n]; }

static int failures = 0;
static void check(bool ok, const char *what, int64_t M, int64_t N, int64_t K, int v, int c) {
    if (!ok && failures++ < 20)
        fprintf(stderr, "plan_driver: %s M=%lld N=%lld K=%lld variant=%d config=%d\n", what, (long long)M,
                (long long)N, (long long)K, v, c);
}

static void check_info(const tlg_plan_info &o, int64_t cap, int64_t M, int64_t N, int64_t K, int v, int c) {
    check(o.grid >= 0 && o.kernels >= 0 && o.kernels <= 2, "grid/kernels", M, N, K, v, c);
    check(o.workspace_bytes >= 0 && o.workspace_bytes <= cap, "workspace within the cap", M, N, K, v, c);
    if (o.variant != TLG_VARIANT_NOOP) check(o.grid > 0 && o.threads > 0, "work-groups", M, N, K, v, c);
    if (o.variant == TLG_VARIANT_NOOP) check(M == 0 || N == 0, "noop only for empty output", M, N, K, v, c);
    check(o.splits >= 1, "splits", M, N, K, v, c);
    check(tlg_plan_config_name(o.variant, o.config) != nullptr, "config name", M, N, K, v, c);
}

int main() {
    const int64_t sizes[] = {0, 1, 2, 7, 8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 255, 256, 257, 1000, 1537,
                             2049, 3001, 4096, 8192, 14336, 65536, 1 << 20, (1ll << 31) - 1025, (1ll << 31) - 1024,
                             1ll << 31, 1ll << 40, -1};
    const int nsizes = sizeof sizes / sizeof sizes[0];
    const int64_t caps[] = {0, 64 << 10, (64 << 10) + 4096, 8 << 20, (8 << 20) + (64 << 10), 32 << 20, 1ll << 40};
    const uintptr_t base16 = 1 << 20, base2 = (1 << 20) + 2;
    int64_t planned = 0;
    for (int t = 0; t < 200000; ++t) {
        const int64_t M = pick(sizes, nsizes), N = pick(sizes, nsizes), K = pick(sizes, nsizes);
        const int64_t pad = (int64_t)(rnd() % 3) * 8 + (int64_t)(rnd() % 2);
        const int64_t lda = (K > 1 ? K : 1) + (rnd() % 4 == 0 ? pad : 0) - (rnd() % 16 == 0 ? 1 : 0);
        const int64_t ldb = (N > 1 ? N : 1) + (rnd() % 4 == 0 ? pad : 0) - (rnd() % 16 == 0 ? 1 : 0);
        const int64_t ldc = (N > 1 ? N : 1) + (rnd() % 4 == 0 ? pad : 0) - (rnd() % 16 == 0 ? 1 : 0);
        const uintptr_t b = rnd() % 2 ? base16 : base2;
        const void *A = (const void *)b, *B = (const void *)(b + 64), *C = (const void *)(b + 128);
        const int v = (int)(rnd() % 11) - 1, c = (int)(rnd() % 18) - 2, s = (int)(rnd() % 22) - 2;
        const int64_t cap = caps[rnd() % (sizeof caps / sizeof caps[0])];
        tlg_plan_info o;
        memset(&o, 0xab, sizeof o);
        const tlg_status ck = tlg_check_args(M, N, K, A, lda, B, ldb, C, ldc);
        const tlg_status st = tlg_plan(M, N, K, A, lda, B, ldb, C, ldc, v, c, s, cap, &o);
        check(st >= TLG_SUCCESS && st <= TLG_ERROR_HIP, "status range", M, N, K, v, c);
        check(tlg_status_string(st) != nullptr, "status string", M, N, K, v, c);
        if (st == TLG_SUCCESS) {
            ++planned;
            check_info(o, cap < (64 << 10) ? (64 << 10) : cap, M, N, K, v, c);
            if (ck != TLG_SUCCESS && !(M == 0 || N == 0)) {
                // tlg_plan checks arguments the same way as the call
            }
        }
        tlg_plan_info ob;
        const tlg_status sb = tlg_plan_bt(M, N, K, A, (K > 1 ? K : 1) + (lda - (K > 1 ? K : 1)), B,
                                          (K > 1 ? K : 1) + (ldb - (N > 1 ? N : 1)), C, ldc, v, c, &ob);
        // the transposed-B call's split strips use the handle's workspace
        if (sb == TLG_SUCCESS) check_info(ob, tlg_workspace_bytes(), M, N, K, v, c);
        const int fmt = (int)(rnd() % 5);
        const int64_t Kx = K >= 0 && rnd() % 2 ? K - K % 32 : K;
        tlg_plan_info om;
        const tlg_status sm = tlg_plan_mx(fmt, M, N, Kx, A, Kx > 1 ? Kx : 1, B, (Kx / 32 > 1 ? Kx / 32 : 1),
                                          (const void *)(b + 256), Kx > 1 ? Kx : 1, (const void *)(b + 512),
                                          (Kx / 32 > 1 ? Kx / 32 : 1), C, ldc, c, &om);
        if (sm == TLG_SUCCESS) check_info(om, 0, M, N, Kx, fmt, c);
        (void)tlg_plan_mx_config_name(c);
    }
    for (int v = -3; v < 12; ++v)
        for (int c = -3; c < 20; ++c) (void)tlg_plan_config_name(v, c);
    for (int st = -2; st < 8; ++st) (void)tlg_status_string((tlg_status)st);
    const char *archs[] = {"gfx950", "gfx950:sramecc+:xnack-", "gfx9500", "", "gfx942", "gfx95"};
    for (const char *a : archs) (void)tlg_arch_supported(a);
    (void)tlg_arch_supported(nullptr);
    check(tlg_workspace_bytes() > 0 && tlg_version() > 0, "constants", 0, 0, 0, 0, 0);
    if (failures) {
        fprintf(stderr, "plan_driver: %d invariant failures\n", failures);
        return 1;
    }
    printf("plan_driver: ok (%lld plans)\n", (long long)planned);
    return 0;
}
