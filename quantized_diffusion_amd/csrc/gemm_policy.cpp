// Host-side choice of the INT8-weight GEMM's output tile (256 x 256 or
// 256 x 384), and the calling thread's setting that can fix it
// (qd_set_gemm_tiles).  Host code only, so that the argument checks of the
// C ABI can be built and tested without the kernels.
#include <stdint.h>

#include "qd_launch.h"

namespace qd {
namespace {

// The kernels' tiles (gemm_i8.hip): 256 activation rows by 256 or 384
// weight rows, K slices of 64 bytes.
constexpr int64_t kTileM = 256, kTileN = 256, kTileNWide = 384, kSliceK = 64;

// The tile setting of the calling thread: one thread's setting never changes
// another thread's launches.
thread_local int g_tile_policy = GEMM_TILES_AUTO;

}  // namespace

void set_gemm_tile_policy(int policy) { g_tile_policy = policy; }

// Cost model for GEMM_TILES_AUTO: rounds of 256 concurrent workgroups (one
// per CU), a round of wide tiles taking 1.41x a round of 256 x 256 tiles
// (1.5x the MACs at the ~6 % better rate measured on M32700/K5376/N16128).
bool gemm_uses_wide_tiles(int64_t M, int64_t N, int64_t K) {
    if (K % kSliceK != 0) return false;
    if (g_tile_policy != GEMM_TILES_AUTO) return g_tile_policy == GEMM_TILES_256x384;
    const int64_t tm = (M + kTileM - 1) / kTileM;
    const int64_t r1 = (tm * ((N + kTileN - 1) / kTileN) + 255) / 256;
    const int64_t r2 = (tm * ((N + kTileNWide - 1) / kTileNWide) + 255) / 256;
    return 141 * r2 < 100 * r1;
}

}  // namespace qd
