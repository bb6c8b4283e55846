// Driver for an AddressSanitizer / UndefinedBehaviorSanitizer build of the
// library's host side (planning, plan checks, workspace sizes and the
// argument checks of every entry point), built from the library's own
// sources with a subset of the kernel shapes (W4A16_VARIANT_SUBSET), the
// sanitizers on host code only, and run where no GPU is visible.  Every call below is answered by host code: the
// pointers are never dereferenced, and a call that passes its checks fails
// the device check.  Exit status 0 means every answer was as expected; the
// sanitizers abort on their own findings.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "w4a16.h"

// a valid call ends at the device check, or (a shape the library was compiled without) at the plan check
static bool device_or_plan(int st) { return st == W4A16_ERR_DEVICE || st == W4A16_ERR_PLAN; }

#define CHECK(c)                                                                 \
    do {                                                                         \
        if (!(c)) {                                                              \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__);  \
            return 1;                                                            \
        }                                                                        \
    } while (0)

int main() {
    void *P = reinterpret_cast<void *>(0x10000), *Q = reinterpret_cast<void *>(0x20000);
    void *odd = reinterpret_cast<void *>(0x10008);
    const int Ks[] = {128, 256, 512, 1280, 5120, 6144, 17408, 1 << 20, 1 << 24};
    const int Ns[] = {16, 48, 528, 1024, 5120, 8192, 34816, 248320};
    long plans = 0;
    for (int M = 1; M <= 16; ++M)
        for (int K : Ks)
            for (int N : Ns) {
                if ((long long)(K / 128) * N * 2 >= (1ll << 31)) {
                    w4a16_plan_t p{};
                    CHECK(w4a16_get_plan(M, N, K, &p) == W4A16_ERR_SHAPE);
                    continue;
                }
                for (int nv = 0; nv < 2; ++nv) {
                    w4a16_plan_t p{};
                    CHECK((nv ? w4a16_nvfp4_get_plan(M, N, K, &p) : w4a16_get_plan(M, N, K, &p)) == W4A16_OK);
                    // built with a subset of the kernel shapes: a plan may name a missing one
                    const int st = nv ? w4a16_nvfp4_check_plan(M, N, K, &p) : w4a16_check_plan(M, N, K, &p);
                    CHECK(st == W4A16_OK || st == W4A16_ERR_PLAN);
                    const size_t ws = nv ? w4a16_nvfp4_workspace_bytes_plan(M, N, K, &p)
                                         : w4a16_workspace_bytes_plan(M, N, K, &p);
                    const size_t any = nv ? w4a16_nvfp4_workspace_bytes(M, N, K) : w4a16_workspace_bytes(M, N, K);
                    CHECK(any >= ws && any >= W4A16_SPLIT_COUNTER_BYTES);
                    ++plans;
                }
            }
    // every plan field out of range is rejected, never crashes
    for (int path = -1; path <= 3; ++path)
        for (int t : {0, 1, 2, 4, 8, 9})
            for (int kw : {0, 1, 4, 8, 17})
                for (int s : {-1, 1, 2, 64})
                    for (int a = -1; a <= 3; ++a)
                        for (int d : {-1, 0, 2, 99})
                            for (int wh : {-1, 0, 40, 1000}) {
                                w4a16_plan_t p{path, t, kw, s, a, d, wh};
                                const int st = w4a16_check_plan(8, 640, 1280, &p);
                                CHECK(st == W4A16_OK || st == W4A16_ERR_PLAN);
                                (void)w4a16_workspace_bytes_plan(8, 640, 1280, &p);
                                (void)w4a16_nvfp4_check_plan(8, 640, 1280, &p);
                            }
    // argument checks of the compute calls (no GPU: valid calls end at the
    // device check).  With a GPU visible they would launch on the fake
    // pointers, so they are left out.
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0) {
        std::printf("host sanitizer check: ok (%ld plans; a GPU is visible, compute-call checks skipped)\n", plans);
        return 0;
    }
    CHECK(w4a16_gemm(nullptr, P, P, Q, 1, 1024, 512, 128, nullptr, 0, nullptr) == W4A16_ERR_NULL);
    CHECK(w4a16_gemm(P, P, P, Q, 17, 1024, 512, 128, nullptr, 0, nullptr) == W4A16_ERR_SHAPE);
    CHECK(w4a16_gemm(P, P, P, Q, 1, 1000, 512, 128, nullptr, 0, nullptr) == W4A16_ERR_SHAPE);
    CHECK(w4a16_gemm(P, P, P, Q, 1, 1024, 512, 64, nullptr, 0, nullptr) == W4A16_ERR_GROUP);
    CHECK(w4a16_gemm(odd, P, P, Q, 1, 1024, 512, 128, nullptr, 0, nullptr) == W4A16_ERR_ALIGN);
    CHECK(device_or_plan(w4a16_gemm(P, P, P, Q, 1, 1024, 512, 128, nullptr, 0, nullptr)));
    CHECK(w4a16_gemm_silu_mul(P, P, P, Q, 1, 1040, 512, 128, nullptr, 0, nullptr) == W4A16_ERR_SHAPE);
    CHECK(w4a16_gemm_argmax(P, P, P, nullptr, nullptr, 1, 1024, 512, 128, nullptr, 0, nullptr) == W4A16_ERR_NULL);
    CHECK(w4a16_gemm_f32(P, P, P, nullptr, 1, 1024, 512, 128, nullptr, 0, nullptr) == W4A16_ERR_NULL);
    CHECK(device_or_plan(w4a16_gemm_noalloc(P, P, P, Q, 1, 1024, 512, 128, nullptr, nullptr)));
    CHECK(w4a16_gemm_noalloc(P, P, P, Q, 0, 1024, 512, 128, nullptr, nullptr) == W4A16_ERR_SHAPE);
    CHECK(w4a16_repack_weights(P, Q, 500, 1024, nullptr) == W4A16_ERR_SHAPE);
    CHECK(w4a16_repack_weights(P, Q, 512, 1024, nullptr) == W4A16_ERR_DEVICE);
    CHECK(w4a16_dequant_debug(P, nullptr, static_cast<float *>(Q), 512, 1024, nullptr) == W4A16_ERR_NULL);
    CHECK(w4a16_nvfp4_gemm(P, P, P, 0.5f, Q, 1, 1024, 512, 128, nullptr, 0, nullptr) == W4A16_ERR_GROUP);
    CHECK(w4a16_nvfp4_repack_scales(odd, Q, 512, 1024, nullptr) == W4A16_ERR_ALIGN);
    for (int st = -9; st <= 0; ++st) CHECK(w4a16_status_string(st) != nullptr);
    CHECK(w4a16_repacked_bytes(5120, 8192) == 5120u * 8192u / 2u);
    std::printf("host sanitizer check: ok (%ld plans)\n", plans);
    return 0;
}
