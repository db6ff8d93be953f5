// qgemm_api.cpp -- the C ABI: argument checks, cached device check, tile
// table, launch.
//
// Boundary conventions follow the caller-owned-output GEMMs of ROCm/aiter PR
// #6262 (Technical Details: out= checked for shape, dtype and device before
// use; the review's request to refuse unsupported layouts) and the tile
// policy of comfy-kitchen PR #174 (Summary: a cached host-side device
// property query picks the tile; an unknown device never reaches a kernel).
// Unlike aiter's A4W4 path, C is exactly [M, N]: edge tiles are masked rather
// than padded to whole 32-row tiles.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/qgemm.h"
#include "qgemm_launch.hpp"
#include "qgemm_pack.hpp"
#include "qgemm_quant.hpp"

using namespace qgemm;

namespace {

thread_local std::string g_last_error;
thread_local int g_forced_tile = -1;

qgemm_status fail(qgemm_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
qgemm_status fail(qgemm_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = std::string(qgemm_status_string(st)) + ": " + buf;
    return st;
}

constexpr int64_t I8_K_MAX = 131071;   // K * 128 * 128 < 2^31
constexpr int64_t LD_LIMIT = (int64_t)1 << 31;

bool aligned(const void *p, unsigned a) { return ((uintptr_t)p & (a - 1)) == 0; }

// ------------------------------------------------------------ device check
// gfx950 or nothing.  The answer per device is cached after the first query.
constexpr int MAX_DEV = 64;
std::once_flag g_dev_once[MAX_DEV];
int g_dev_ok[MAX_DEV];

bool is_gfx950(const char *name)
{
    return strncmp(name, "gfx950", 6) == 0 && (name[6] == 0 || name[6] == ':');
}

// Test hook: QGEMM_INJECT_LAUNCH_ERROR=<hipError_t code> makes every call
// that passed its checks report that launch error (QGEMM_ERR_HIP) instead of
// launching, so the error path can be exercised without a failing GPU.
int injected_launch_error()
{
    const char *v = getenv("QGEMM_INJECT_LAUNCH_ERROR");
    return (v && *v) ? atoi(v) : 0;
}

qgemm_status check_device()
{
    // Test hooks: a fake architecture name that is not gfx950 is refused
    // before any HIP call is made; a fake gfx950 is accepted without one, but
    // only while a launch error is injected (nothing can reach a kernel).
    const char *fake = getenv("QGEMM_FAKE_ARCH");
    if (fake && *fake && !is_gfx950(fake))
        return fail(QGEMM_ERR_UNSUPPORTED_DEVICE, "device reports %s, not gfx950", fake);
    if (fake && *fake && injected_launch_error())
        return QGEMM_OK;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(QGEMM_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= MAX_DEV)
        return fail(QGEMM_ERR_UNSUPPORTED_DEVICE, "device index %d out of range", dev);
    std::call_once(g_dev_once[dev], [dev]() {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            g_dev_ok[dev] = -1;
            return;
        }
        g_dev_ok[dev] = is_gfx950(prop.gcnArchName) ? 1 : 0;
    });
    if (g_dev_ok[dev] == 1)
        return QGEMM_OK;
    if (g_dev_ok[dev] < 0)
        return fail(QGEMM_ERR_HIP, "hipGetDeviceProperties failed for device %d", dev);
    return fail(QGEMM_ERR_UNSUPPORTED_DEVICE, "device %d is not gfx950", dev);
}

// ------------------------------------------------------------ tile table
// A launch runs in rounds of (CUs x workgroups per CU) tiles; a round lasts
// about as long as one workgroup's tile at its measured MFMA efficiency, times
// the workgroups that share a CU (none while the grid is smaller than the
// chip).  The table picks the candidate with
// the smallest rounds x round-time; ties keep the earlier (larger) tile.  The
// efficiencies are relative figures from the benchmark workloads: the 192x192
// tile moves ~1.3x the LDS bytes per MFMA of the 256x256 tile, the 128x128
// tile ~2x.
struct TileCand {
    int tile;
    int per_cu;      // workgroups resident per CU (LDS and registers)
    double eff;      // MFMA efficiency relative to the 256x256 tile
};
const TileCand TILE_TABLE[] = {
    {0, 1, 1.00},   // 256x256, 4 waves, 128 KB LDS
    {3, 1, 0.85},   // 192x192, 4 waves, 96 KB LDS
    {1, 2, 0.55},   // 128x128, 4 waves, 64 KB LDS: two per CU
};
constexpr int NUM_CU = 256;
constexpr double MALL_BYTES = 256.0 * 1024 * 1024;   // MI355X Infinity Cache

int select_tile_impl(int path, int64_t M, int64_t N)
{
    (void)path;
    int best = TILE_TABLE[0].tile;
    double best_cost = -1.0;
    for (const TileCand &c : TILE_TABLE) {
        const int64_t e = tile_edge(c.tile);
        const int64_t tiles = ((M + e - 1) / e) * ((N + e - 1) / e);
        const int64_t slots = (int64_t)NUM_CU * c.per_cu;
        const int64_t rounds = (tiles + slots - 1) / slots;
        // workgroups that actually share a CU: none while the grid is smaller
        // than the chip
        const int64_t share = std::min<int64_t>(c.per_cu, (tiles + NUM_CU - 1) / NUM_CU);
        const double cost = (double)rounds * (double)(e * e) * (double)share / c.eff;
        if (best_cost < 0 || cost < best_cost * 0.999) {
            best = c.tile;
            best_cost = cost;
        }
    }
    return best;
}

// ------------------------------------------------------------ common checks
struct Shape {
    int64_t M, N, K;
};

qgemm_status check_shape(Shape s, bool is_i8)
{
    if (s.M < 0 || s.N < 0 || s.K <= 0)
        return fail(QGEMM_ERR_BAD_SHAPE, "M=%lld N=%lld K=%lld: need M>=0, N>=0, K>0", (long long)s.M,
                    (long long)s.N, (long long)s.K);
    if (s.K % 32)
        return fail(QGEMM_ERR_BAD_SHAPE, "K=%lld is not a multiple of 32", (long long)s.K);
    if (s.M >= LD_LIMIT || s.N >= LD_LIMIT || s.K >= LD_LIMIT)
        return fail(QGEMM_ERR_BAD_SHAPE, "M, N and K must stay below 2^31");
    if (is_i8 && s.K > I8_K_MAX)
        return fail(QGEMM_ERR_BAD_SHAPE, "K=%lld exceeds %lld (int32 accumulator range)", (long long)s.K,
                    (long long)I8_K_MAX);
    return QGEMM_OK;
}

qgemm_status check_operand(const char *name, const void *p, int64_t ld, int64_t row_bytes)
{
    if (!p)
        return fail(QGEMM_ERR_NULL_POINTER, "%s is NULL", name);
    if (!aligned(p, 16))
        return fail(QGEMM_ERR_BAD_LAYOUT, "%s is not 16-byte aligned", name);
    if (ld < row_bytes)
        return fail(QGEMM_ERR_BAD_LAYOUT, "ld%s=%lld bytes is below the row (%lld bytes)", name, (long long)ld,
                    (long long)row_bytes);
    if (ld % 16)
        return fail(QGEMM_ERR_BAD_LAYOUT, "ld%s=%lld is not a multiple of 16 bytes", name, (long long)ld);
    if (ld * 256 >= LD_LIMIT)
        return fail(QGEMM_ERR_BAD_LAYOUT, "ld%s=%lld bytes: 256 rows exceed 2^31 bytes", name, (long long)ld);
    return QGEMM_OK;
}

qgemm_status check_output(const void *C, int64_t ldc, int64_t N, int esz)
{
    if (!C)
        return fail(QGEMM_ERR_NULL_POINTER, "C is NULL");
    if (!aligned(C, 16))
        return fail(QGEMM_ERR_BAD_LAYOUT, "C is not 16-byte aligned");
    if (ldc < N)
        return fail(QGEMM_ERR_BAD_LAYOUT, "ldc=%lld is below N=%lld", (long long)ldc, (long long)N);
    if (ldc % 8)
        return fail(QGEMM_ERR_BAD_LAYOUT, "ldc=%lld is not a multiple of 8", (long long)ldc);
    if (ldc * esz * 256 >= LD_LIMIT)
        return fail(QGEMM_ERR_BAD_LAYOUT, "ldc=%lld: 256 rows exceed 2^31 bytes", (long long)ldc);
    return QGEMM_OK;
}

qgemm_status check_fp32_scales(const float *sa, const float *sb)
{
    if (!sa)
        return fail(QGEMM_ERR_NULL_POINTER, "scale_a is NULL");
    if (!sb)
        return fail(QGEMM_ERR_NULL_POINTER, "scale_b is NULL");
    if (!aligned(sa, 4) || !aligned(sb, 4))
        return fail(QGEMM_ERR_BAD_LAYOUT, "fp32 scales must be 4-byte aligned");
    return QGEMM_OK;
}

qgemm_status check_bias(const uint16_t *bias)
{
    if (bias && !aligned(bias, 2))
        return fail(QGEMM_ERR_BAD_LAYOUT, "bias is not 2-byte aligned");
    return QGEMM_OK;
}

#define TRY(x)                                  \
    do {                                        \
        qgemm_status st_ = (x);                 \
        if (st_ != QGEMM_OK)                    \
            return st_;                         \
    } while (0)

Params base_params(const void *A, int64_t lda, const void *B, int64_t ldb, void *C, int64_t ldc, Shape s,
                   int64_t kbytes, int tile)
{
    Params p;
    memset(&p, 0, sizeof p);
    p.A = (const uint8_t *)A;
    p.B = (const uint8_t *)B;
    p.lda = lda;
    p.ldb = ldb;
    p.C = C;
    p.ldc = ldc;
    p.M = (int)s.M;
    p.N = (int)s.N;
    p.K = (int)s.K;
    p.kbytes = (int)kbytes;
    p.ksteps = (int)((kbytes + KSTEP_BYTES - 1) / KSTEP_BYTES);
    p.kblocks = (int)(s.K / 32);
    const int em = tile_edge_m(tile), en = tile_edge_n(tile);
    p.tiles_m = (int)((s.M + em - 1) / em);
    p.tiles_n = (int)((s.N + en - 1) / en);
    // small-M tiles: every row tile of one column block runs next to the others
    p.group_m = is_skinny_tile(tile) ? p.tiles_m : 8;
    // Output stores: through the caches when C, A and B together fit the
    // 256 MB MALL (the output then stays there for whoever reads it next, and
    // the write burst at the end of each round of tiles drains behind the next
    // round: MXFP4 8192^3, 201 MB, 0.272 -> 0.262 ms), non-temporal otherwise
    // (where C would only push the operands out: INT8 30000x21504x5376 2.84
    // vs 2.93 ms, MXFP8 16384x7168x2048 0.236 vs 0.240 ms; one MI355X, same
    // machine alternating).
    const double footprint = (double)s.M * (double)s.N * 2.0 + (double)(s.M + s.N) * (double)kbytes;
    p.c_cached = footprint <= MALL_BYTES ? 1 : 0;
    return p;
}

qgemm_status check_grid(const Params &p)
{
    if ((int64_t)p.tiles_m * p.tiles_n >= LD_LIMIT)
        return fail(QGEMM_ERR_BAD_SHAPE, "grid of %d x %d tiles is too large", p.tiles_m, p.tiles_n);
    return QGEMM_OK;
}

qgemm_status finish(hipError_t e)
{
    if (e != hipSuccess)
        return fail(QGEMM_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
    return QGEMM_OK;
}

// Every launch goes through here: the kernel launch (f), or the injected
// launch error, which leaves the output and everything else untouched.
template <class F>
qgemm_status launch(F &&f)
{
    if (const int e = injected_launch_error())
        return fail(QGEMM_ERR_HIP, "kernel launch: injected error %d", e);
    return finish(f());
}

// The LDS-fetch kernels (tiles 4-7) run tiles whose K is a whole number of
// their 64-byte stages (a last round of fewer than four is masked).  For MX,
// a round reads 16 bytes of each scale row from byte 16u (e2m1) or 8u (e4m3),
// from the row's start rounded down to a dword (a whole dword unless K % 128
// != 0), and the caller's scale arrays aligned to 16 / 8 bytes (svec: the
// caller's check).
//
// The masked last round keeps word 0 of a round's scale chunk live and
// replaces later words past K; a word covers 4 / (words per round) stages.
// e2m1 (one stage per word) needs K % 128 for whole 64-byte stages, the
// blockscale and 6-bit paths K % 128 by their blocks and rows.  The
// e4m3-staged MX paths (e4m3, and both mixed pairings: 64 K elements a stage,
// two stages per word) take any K % 32: at K % 128 != 0 their scale rows
// start off dword boundaries, the last live word may end part way past K
// and, at K % 64 == 32, the last stage half way, which the LDS-fetch
// kernel's SU form handles (fetches from the start rounded down to a dword,
// byte masking of the scale words, the half stage's other chunks fetched as
// zeros).  dma_k_ok is the one place that rule lives; every LDS-fetch path
// takes it.
bool dma_k_ok(int path, int64_t K)
{
    switch (path) {
    case 0:
    case 1: return K % 64 == 0;    // int8 / e4m3 bytes: whole 64-byte stages
    case 2:                        // e4m3 MX
    case 5:                        // mixed MX, e4m3 A x e2m1 B
    case 8: return K % 32 == 0;    // mixed MX, e2m1 A x e4m3 B
    default: return K % 128 == 0;  // e2m1, blockscale, 6-bit: whole scale words per round
    }
}

bool dma_eligible(int path, int64_t kbytes, int64_t K, bool svec)
{
    if ((path == 2 || path == 3) && !svec)
        return false;
    const bool e4m3_staged = path == 2 || path == 5 || path == 8;   // K % 32: the SU form
    return (e4m3_staged || kbytes % 64 == 0) && dma_k_ok(path, K);
}

// When K fits, the table's tile edge runs in an LDS-fetch kernel: 256 as the
// eight-wave kernel (one MI355X, same machine: INT8 30000x21504x5376 2155 TOPS vs
// 2130 for the four-wave LDS-fetch kernel and ~2100 for register staging;
// MXFP4 8192^3 3756 vs 3668 TFLOPS; MXFP8 16384x7168x2048 1940 vs 1933), 192
// and 128 as their four-wave LDS-fetch forms.
// Small M (bf16 output): the call streams B; the small-M kernel spreads B
// over N/16 workgroups whose eight waves split K.  MX only up to 16 rows: its
// 64-row form loses to the 128x128 LDS-fetch tile (one MI355X, MXFP8
// 64x7168x2048: 19.9 vs 13.1 us; MXFP4 64x8192x8192: 43 vs 23.5 us), while
// the 16-row form wins (MXFP8 1x7168x2048 8.0 vs 9.5 us, MXFP4 1x8192x8192
// 13.5 vs 18.3 us).
constexpr int64_t SKINNY_MAX_M = 64, SKINNY_MAX_M_MX = 16;

// The LDS-fetch form of the 256x256 edge: the eight-wave kernel, whose INT8
// and e2m1 forms fetch two stages of a row per request (one MI355X, same machine
// alternating: INT8 30000x21504x5376 2.909 ms on tile 5 vs 3.031 ms on the
// four-wave tile 4; MXFP4 8192^3 0.304 vs 0.332 ms; MXFP8 16384x7168x2048
// 0.248 vs 0.255 ms) -- except INT8 with a prepacked B, whose whole-line
// fetches gain nothing from pairs and keep the four-wave kernel's deeper
// prefetch (2.862 vs 2.900 ms).
int big_dma_tile(int path, bool packed = false) { return (path == 0 && packed) ? DMA_TILE : DMA8_TILE; }

int pick_tile(int path, Shape s, int64_t kbytes, bool svec, bool bf16_out)
{
    const bool skinny_ok = bf16_out;
    int t;
    if (g_forced_tile >= 0) {
        t = g_forced_tile;
    } else if (skinny_ok && s.M <= (path >= 2 ? SKINNY_MAX_M_MX : SKINNY_MAX_M)) {
        t = s.M <= 16 ? SKINNY16_TILE : SKINNY64_TILE;
    } else {
        t = select_tile_impl(path, s.M, s.N);
        if (dma_eligible(path, kbytes, s.K, svec))
            t = (t == 0) ? big_dma_tile(path) : (t == 3) ? DMA192_TILE : (t == 1) ? DMA128_TILE : t;
    }
    if (t == F8B256_TILE)   // a blockscale-only tile, forced on another path
        t = 0;
    if (is_dma_tile(t) && !dma_eligible(path, kbytes, s.K, svec))
        t = 0;
    if (is_skinny_tile(t) && !skinny_ok)
        t = 0;
    return t;
}

// A prepacked B is read only by the LDS-fetch and small-M kernels (the caller
// checked that K fits them): a forced register-staged tile runs as the
// LDS-fetch kernel of its edge, and the table's choice as for row-major B.
int pick_tile_packed(int path, Shape s, int64_t kbytes, bool bf16_out)
{
    const int t = pick_tile(path, s, kbytes, true, bf16_out);
    if (g_forced_tile < 0 && t == big_dma_tile(path))
        return big_dma_tile(path, true);
    switch (t) {
    case 0: return g_forced_tile == 0 ? DMA_TILE : big_dma_tile(path, true);
    case 1: return DMA128_TILE;
    case 2: return DMA8_TILE;
    case 3: return DMA192_TILE;
    default: return t;
    }
}

// Blockscale FP8 runs in the LDS-fetch kernel: K must be a whole number of
// 128-element blocks (two stages); a round reads 8 bytes (two K blocks) of
// every scale row, a last round of one block masks the other.  A prepacked B
// keeps the packer's K % 256.  The 256x128 tile (one workgroup per CU) when its grid
// fills the chip at least once, else the 128x128 tile (two per CU, half the
// rows): one MI355X, 16384x7168x2048 0.302 ms vs 0.310 ms.
constexpr int64_t F8B_K_MULTIPLE = 128;

// Mixed MX (e4m3 A, e2m1 B) runs in the LDS-fetch kernel: 256x256 (tile 4,
// or 5 when forced) or 128x128 (tile 7) -- the table's 192x192 choice takes
// tile 7 -- and for M <= 16 in the small-M kernel (tile 8; 9 when forced).
int pick_tile_mx84(Shape s)
{
    if (g_forced_tile == DMA_TILE || g_forced_tile == DMA8_TILE || g_forced_tile == DMA128_TILE ||
        g_forced_tile == SKINNY16_TILE || g_forced_tile == SKINNY64_TILE)
        return g_forced_tile;
    if (s.M <= SKINNY_MAX_M_MX)
        return SKINNY16_TILE;
    // the four-wave 256x256 tile, where the 16-byte wide scale refills apply
    // (8192^3 on one machine, alternating: 0.445 vs 0.477 ms for the eight-wave
    // tile 5)
    return select_tile_impl(2, s.M, s.N) == 0 ? DMA_TILE : DMA128_TILE;
}

// Mixed MX the other way round (e2m1 A, e4m3 B): the LDS-fetch kernel only,
// 256x256 (tile 4, or 5 when forced) where the 256x256 grid fills the chip,
// else 128x128 (tile 7), small M included (no small-M form).
int pick_tile_mx48(Shape s)
{
    if (g_forced_tile == DMA_TILE || g_forced_tile == DMA8_TILE || g_forced_tile == DMA128_TILE)
        return g_forced_tile;
    return select_tile_impl(2, s.M, s.N) == 0 ? DMA_TILE : DMA128_TILE;
}

// e2m1 MX at K % 128 != 0 (K/32 not a multiple of 4): the LDS-fetch kernel
// in 64-element stages -- the eight-wave tile 5 where the table picks 256x256
// (one MI355X, 8192x8192x8256: 0.505 ms against 0.551 on tile 4 and 0.799 on
// the register-staged tile), else 7 (forced: 4, 5, 7) -- unless the call
// takes the small-M kernel (M <= 16, or forced 8 / 9) or a forced
// register-staged tile: then -1, the e2m1 path's own choice.
int pick_tile_mx4h(Shape s)
{
    if (g_forced_tile == DMA_TILE || g_forced_tile == DMA8_TILE || g_forced_tile == DMA128_TILE)
        return g_forced_tile;
    if (g_forced_tile >= 0 || s.M <= SKINNY_MAX_M_MX)
        return -1;
    return select_tile_impl(3, s.M, s.N) == 0 ? DMA8_TILE : DMA128_TILE;
}

// 6-bit MX: the four-wave 256x256 tile where the 256x256 grid fills the
// chip, else 128x128 (the only two FP6 tiles built).
int pick_tile_mx6(Shape s)
{
    if (g_forced_tile == DMA_TILE || g_forced_tile == DMA128_TILE)
        return g_forced_tile;
    return select_tile_impl(3, s.M, s.N) == 0 ? DMA_TILE : DMA128_TILE;
}

int pick_tile_f8b(int64_t M, int64_t N)
{
    if (g_forced_tile == F8B256_TILE || g_forced_tile == DMA128_TILE || g_forced_tile == SKINNY16_TILE ||
        g_forced_tile == SKINNY64_TILE)
        return g_forced_tile;
    if (M <= SKINNY_MAX_M_MX)   // small M: the small-M kernel, one 16-row block
        return SKINNY16_TILE;
    return ((M + 255) / 256) * ((N + 127) / 128) >= NUM_CU ? F8B256_TILE : DMA128_TILE;
}

}  // namespace

extern "C" {

const char *qgemm_status_string(qgemm_status st)
{
    switch (st) {
    case QGEMM_OK: return "QGEMM_OK";
    case QGEMM_ERR_NULL_POINTER: return "QGEMM_ERR_NULL_POINTER";
    case QGEMM_ERR_BAD_SHAPE: return "QGEMM_ERR_BAD_SHAPE";
    case QGEMM_ERR_BAD_LAYOUT: return "QGEMM_ERR_BAD_LAYOUT";
    case QGEMM_ERR_BAD_FORMAT: return "QGEMM_ERR_BAD_FORMAT";
    case QGEMM_ERR_UNSUPPORTED_DEVICE: return "QGEMM_ERR_UNSUPPORTED_DEVICE";
    case QGEMM_ERR_HIP: return "QGEMM_ERR_HIP";
    }
    return "QGEMM_UNKNOWN_STATUS";
}

const char *qgemm_last_error(void) { return g_last_error.c_str(); }

int qgemm_select_tile(int path, int64_t M, int64_t N, int64_t K)
{
    if (path < 0 || path > 8)
        return -1;
    if (path == 8) {   // MX e2m1 A x e4m3 B
        const int prev = g_forced_tile;
        g_forced_tile = -1;
        const int t = pick_tile_mx48(Shape{M, N, K});
        g_forced_tile = prev;
        return t;
    }
    if (path == 6 || path == 7) {   // MX e2m3 / e3m2
        const int prev = g_forced_tile;
        g_forced_tile = -1;
        const int t = pick_tile_mx6(Shape{M, N, K});
        g_forced_tile = prev;
        return t;
    }
    if (path == 5) {   // MX e4m3 A x e2m1 B
        const int prev = g_forced_tile;
        g_forced_tile = -1;
        const int t = pick_tile_mx84(Shape{M, N, K});
        g_forced_tile = prev;
        return t;
    }
    if (path == 4) {
        const int prev = g_forced_tile;
        g_forced_tile = -1;
        const int t = pick_tile_f8b(M, N);
        g_forced_tile = prev;
        return t;
    }
    const int64_t kbytes = path == 3 ? K / 2 : K;
    const int prev = g_forced_tile;
    g_forced_tile = -1;
    int t = (path == 3 && K % 128 != 0) ? pick_tile_mx4h(Shape{M, N, K}) : -1;
    if (t < 0)
        t = pick_tile(path, Shape{M, N, K}, kbytes, true, true);   // scales assumed aligned, bf16 out
    g_forced_tile = prev;
    return t;
}

int qgemm_tile_rows(int tile) { return (tile >= 0 && tile < NUM_TILES) ? tile_edge(tile) : 0; }

int qgemm_force_tile(int tile)
{
    if (tile < -1 || tile >= NUM_TILES)
        return -2;
    const int prev = g_forced_tile;
    g_forced_tile = tile;
    return prev;
}

// A prepacked B (qgemm_prepack_b's layout): 16-byte aligned, row bytes a
// whole number of the LDS-fetch kernel's 4 x 64-byte stage rounds.
static qgemm_status check_packed_b(const void *Bp, int64_t row_bytes)
{
    if (!Bp)
        return fail(QGEMM_ERR_NULL_POINTER, "Bp is NULL");
    if (!aligned(Bp, 16))
        return fail(QGEMM_ERR_BAD_LAYOUT, "Bp is not 16-byte aligned");
    if (row_bytes % 256)
        return fail(QGEMM_ERR_BAD_SHAPE, "a prepacked B needs rows of a multiple of 256 bytes, got %lld",
                    (long long)row_bytes);
    if (row_bytes * 256 >= LD_LIMIT)
        return fail(QGEMM_ERR_BAD_SHAPE, "rows of %lld bytes: 256 rows exceed 2^31 bytes", (long long)row_bytes);
    return QGEMM_OK;
}

static qgemm_status i8_common(const int8_t *A, int64_t lda, const void *B, int64_t ldb, const float *sa,
                              const float *sb, const uint16_t *bias, void *C, int64_t ldc, Shape s, void *stream,
                              int out, bool packed = false)
{
    TRY(check_shape(s, true));
    if (s.M == 0 || s.N == 0)
        return QGEMM_OK;
    TRY(check_operand("A", A, lda, s.K));
    if (packed)
        TRY(check_packed_b(B, s.K));
    else
        TRY(check_operand("B", B, ldb, s.K));
    if (out == OUT_BF16) {
        TRY(check_fp32_scales(sa, sb));
        TRY(check_bias(bias));
    }
    TRY(check_output(C, ldc, s.N, out == OUT_I32 ? 4 : 2));
    TRY(check_device());
    const int tile = packed ? pick_tile_packed(0, s, s.K, out == OUT_BF16) : pick_tile(0, s, s.K, true, out == OUT_BF16);
    Params p = base_params(A, lda, B, packed ? s.K : ldb, C, ldc, s, s.K, tile);
    p.b_packed = packed;
    TRY(check_grid(p));
    p.scale_a = sa;
    p.scale_b = sb;
    p.bias = bias;
    return launch([&] { return launch_i8(tile, bias != nullptr, out, p, (hipStream_t)stream); });
}

qgemm_status qgemm_i8_rowwise(const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb, const float *scale_a,
                              const float *scale_b, const uint16_t *bias, uint16_t *C, int64_t ldc, int64_t M,
                              int64_t N, int64_t K, void *stream)
{
    return i8_common(A, lda, B, ldb, scale_a, scale_b, bias, C, ldc, Shape{M, N, K}, stream, OUT_BF16);
}

qgemm_status qgemm_i8_acc_i32(const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb, int32_t *C,
                              int64_t ldc, int64_t M, int64_t N, int64_t K, void *stream)
{
    return i8_common(A, lda, B, ldb, nullptr, nullptr, nullptr, C, ldc, Shape{M, N, K}, stream, OUT_I32);
}

static qgemm_status f8_common(const uint8_t *A, int64_t lda, const void *B, int64_t ldb, const float *scale_a,
                              const float *scale_b, const uint16_t *bias, uint16_t *C, int64_t ldc, int64_t M,
                              int64_t N, int64_t K, void *stream, bool packed)
{
    const Shape s{M, N, K};
    TRY(check_shape(s, false));
    if (M == 0 || N == 0)
        return QGEMM_OK;
    TRY(check_operand("A", A, lda, K));
    if (packed)
        TRY(check_packed_b(B, K));
    else
        TRY(check_operand("B", B, ldb, K));
    TRY(check_fp32_scales(scale_a, scale_b));
    TRY(check_bias(bias));
    TRY(check_output(C, ldc, N, 2));
    TRY(check_device());
    const int tile = packed ? pick_tile_packed(1, s, K, true) : pick_tile(1, s, K, true, true);
    Params p = base_params(A, lda, B, packed ? K : ldb, C, ldc, s, K, tile);
    p.b_packed = packed;
    TRY(check_grid(p));
    p.scale_a = scale_a;
    p.scale_b = scale_b;
    p.bias = bias;
    return launch([&] { return launch_f8(tile, bias != nullptr, p, (hipStream_t)stream); });
}

qgemm_status qgemm_f8_pertoken(const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb, const float *scale_a,
                               const float *scale_b, const uint16_t *bias, uint16_t *C, int64_t ldc, int64_t M,
                               int64_t N, int64_t K, void *stream)
{
    return f8_common(A, lda, B, ldb, scale_a, scale_b, bias, C, ldc, M, N, K, stream, false);
}

static qgemm_status f8b_common(const uint8_t *A, int64_t lda, const void *B, int64_t ldb, const float *scale_a,
                               const float *scale_b, const uint16_t *bias, uint16_t *C, int64_t ldc, int64_t M,
                               int64_t N, int64_t K, void *stream, bool packed)
{
    const Shape s{M, N, K};
    TRY(check_shape(s, false));
    if (!dma_k_ok(4, K))
        return fail(QGEMM_ERR_BAD_SHAPE, "K=%lld: blockscale needs K a multiple of %lld", (long long)K,
                    (long long)F8B_K_MULTIPLE);
    if (M == 0 || N == 0)
        return QGEMM_OK;
    TRY(check_operand("A", A, lda, K));
    if (packed)
        TRY(check_packed_b(B, K));
    else
        TRY(check_operand("B", B, ldb, K));
    TRY(check_fp32_scales(scale_a, scale_b));
    if (!aligned(scale_a, 8) || !aligned(scale_b, 8))
        return fail(QGEMM_ERR_BAD_LAYOUT, "blockscale scale arrays must be 8-byte aligned");
    TRY(check_bias(bias));
    TRY(check_output(C, ldc, N, 2));
    TRY(check_device());
    const int tile = pick_tile_f8b(M, N);
    Params p = base_params(A, lda, B, packed ? K : ldb, C, ldc, s, K, tile);
    p.b_packed = packed;
    TRY(check_grid(p));
    // the scale matrices travel as byte rows of K/32 bytes (K/128 floats)
    p.mx_sa = (const uint8_t *)scale_a;
    p.mx_sb = (const uint8_t *)scale_b;
    p.bias = bias;
    return launch([&] { return launch_f8b(tile, bias != nullptr, p, (hipStream_t)stream); });
}

qgemm_status qgemm_f8_blockscale(const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb, const float *scale_a,
                                 const float *scale_b, const uint16_t *bias, uint16_t *C, int64_t ldc, int64_t M,
                                 int64_t N, int64_t K, void *stream)
{
    return f8b_common(A, lda, B, ldb, scale_a, scale_b, bias, C, ldc, M, N, K, stream, false);
}

// MX with 6-bit elements: rows of 3K/4 bytes, the LDS-fetch kernel's 48-byte
// stages of 64 elements and the e4m3 scale staging (8 bytes of each scale
// row per round, so 8-byte aligned scale arrays).
static qgemm_status mx6_common(qgemm_mx_fmt fmt, const void *A, int64_t lda_bytes, const void *B, int64_t ldb_bytes,
                               const uint8_t *scale_a, const uint8_t *scale_b, qgemm_mx_bscale b_layout,
                               const uint16_t *bias, uint16_t *C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                               void *stream)
{
    const Shape s{M, N, K};
    TRY(check_shape(s, false));
    if (!dma_k_ok(6, K))
        return fail(QGEMM_ERR_BAD_SHAPE, "K=%lld: 6-bit MX needs K a multiple of 128", (long long)K);
    if (M == 0 || N == 0)
        return QGEMM_OK;
    const int64_t row_bytes = 3 * K / 4;
    TRY(check_operand("A", A, lda_bytes, row_bytes));
    TRY(check_operand("B", B, ldb_bytes, row_bytes));
    if (!scale_a)
        return fail(QGEMM_ERR_NULL_POINTER, "scale_a is NULL");
    if (!scale_b)
        return fail(QGEMM_ERR_NULL_POINTER, "scale_b is NULL");
    if (!aligned(scale_a, 8) || !aligned(scale_b, 8))
        return fail(QGEMM_ERR_BAD_LAYOUT, "6-bit MX scale arrays must be 8-byte aligned");
    TRY(check_bias(bias));
    TRY(check_output(C, ldc, N, 2));
    TRY(check_device());
    const int tile = pick_tile_mx6(s);
    Params p = base_params(A, lda_bytes, B, ldb_bytes, C, ldc, s, row_bytes, tile);
    TRY(check_grid(p));
    p.mx_sa = scale_a;
    p.mx_sb = scale_b;
    p.bias = bias;
    return launch([&] { return launch_mx6(tile, fmt == QGEMM_MX_E3M2, bias != nullptr, (int)b_layout, p, (hipStream_t)stream); });
}

static qgemm_status mx_common(qgemm_mx_fmt fmt, const void *A, int64_t lda_bytes, const void *B, int64_t ldb_bytes,
                              const uint8_t *scale_a, const uint8_t *scale_b, qgemm_mx_bscale b_layout,
                              const uint16_t *bias, uint16_t *C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                              void *stream, bool packed)
{
    const Shape s{M, N, K};
    if (fmt != QGEMM_MX_E4M3 && fmt != QGEMM_MX_E2M1 && fmt != QGEMM_MX_E2M3 && fmt != QGEMM_MX_E3M2)
        return fail(QGEMM_ERR_BAD_FORMAT, "unknown MX element format %d", (int)fmt);
    if (b_layout != QGEMM_MX_BSCALE_1x32 && b_layout != QGEMM_MX_BSCALE_32x32)
        return fail(QGEMM_ERR_BAD_FORMAT, "unknown B-scale layout %d", (int)b_layout);
    if (fmt == QGEMM_MX_E2M3 || fmt == QGEMM_MX_E3M2)
        return packed ? fail(QGEMM_ERR_BAD_FORMAT, "no prepacked layout for 6-bit MX elements")
                      : mx6_common(fmt, A, lda_bytes, B, ldb_bytes, scale_a, scale_b, b_layout, bias, C, ldc, M, N,
                                   K, stream);
    TRY(check_shape(s, false));
    if (M == 0 || N == 0)
        return QGEMM_OK;
    const int64_t row_bytes = (fmt == QGEMM_MX_E4M3) ? K : K / 2;
    TRY(check_operand("A", A, lda_bytes, row_bytes));
    if (packed)
        TRY(check_packed_b(B, row_bytes));
    else
        TRY(check_operand("B", B, ldb_bytes, row_bytes));
    if (!scale_a)
        return fail(QGEMM_ERR_NULL_POINTER, "scale_a is NULL");
    if (!scale_b)
        return fail(QGEMM_ERR_NULL_POINTER, "scale_b is NULL");
    TRY(check_bias(bias));
    TRY(check_output(C, ldc, N, 2));
    const int path = (fmt == QGEMM_MX_E4M3) ? 2 : 3;
    // Scale words load whole when every lane's bytes of a K step are aligned:
    // e2m1 takes 4 bytes per lane half (K/32 % 4 == 0), e4m3 takes 2 (K/32 even),
    // and the scale arrays themselves start aligned.  The LDS-fetch kernel
    // reads 16 (e2m1) or 8 (e4m3) bytes of each scale row per round: the
    // arrays must be aligned to that.
    // sdma: the scales fit the LDS-fetch kernel (e4m3 at any K/32: its SU
    // form; the register-staged tile then loads scale bytes)
    const int wb = (fmt == QGEMM_MX_E2M1) ? 4 : 2;
    const bool svec = ((K / 32) % wb == 0) && aligned(scale_a, wb) && aligned(scale_b, wb);
    const unsigned chunk_align = (fmt == QGEMM_MX_E2M1) ? 16 : 8;
    const bool sdma = (svec || fmt == QGEMM_MX_E4M3) && aligned(scale_a, chunk_align) && aligned(scale_b, chunk_align);
    if (packed && (row_bytes % 256 || !dma_eligible(path, row_bytes, K, sdma)))
        return fail(QGEMM_ERR_BAD_LAYOUT, "a prepacked MX B needs K/32 a multiple of 16 (e2m1) or 8 (e4m3) and scale "
                                          "arrays aligned to 16 (e2m1) or 8 (e4m3) bytes");
    TRY(check_device());
    if (fmt == QGEMM_MX_E2M1 && !packed && K % 128 != 0 && aligned(scale_a, 8) && aligned(scale_b, 8)) {
        const int t4 = pick_tile_mx4h(s);
        if (t4 >= 0) {
            Params p = base_params(A, lda_bytes, B, ldb_bytes, C, ldc, s, K, t4);   // kbytes: K, as for e4m3
            TRY(check_grid(p));
            p.mx_sa = scale_a;
            p.mx_sb = scale_b;
            p.bias = bias;
            return launch([&] { return launch_mx4h(t4, bias != nullptr, (int)b_layout, p, (hipStream_t)stream); });
        }
    }
    const int tile = packed ? pick_tile_packed(path, s, row_bytes, true) : pick_tile(path, s, row_bytes, sdma, true);
    Params p = base_params(A, lda_bytes, B, packed ? row_bytes : ldb_bytes, C, ldc, s, row_bytes, tile);
    p.b_packed = packed;
    TRY(check_grid(p));
    p.mx_sa = scale_a;
    p.mx_sb = scale_b;
    p.bias = bias;
    const int brows = (int)b_layout;
    if (fmt == QGEMM_MX_E4M3)
        return launch([&] { return launch_mx8(tile, bias != nullptr, brows, svec, p, (hipStream_t)stream); });
    return launch([&] { return launch_mx4(tile, bias != nullptr, brows, svec, p, (hipStream_t)stream); });
}

static qgemm_status mx_mixed_common(qgemm_mx_fmt fmt_a, qgemm_mx_fmt fmt_b, const void *A, int64_t lda_bytes,
                                    const void *B, int64_t ldb_bytes, const uint8_t *scale_a, const uint8_t *scale_b,
                                    qgemm_mx_bscale b_layout, const uint16_t *bias, uint16_t *C, int64_t ldc,
                                    int64_t M, int64_t N, int64_t K, void *stream, bool packed)
{
    const bool known_a = fmt_a == QGEMM_MX_E4M3 || fmt_a == QGEMM_MX_E2M1;
    const bool known_b = fmt_b == QGEMM_MX_E4M3 || fmt_b == QGEMM_MX_E2M1;
    if (!known_a || !known_b)
        return fail(QGEMM_ERR_BAD_FORMAT, "unknown MX element format %d / %d", (int)fmt_a, (int)fmt_b);
    if (fmt_a == fmt_b) {
        if (packed)
            return fail(QGEMM_ERR_BAD_FORMAT, "equal formats: use qgemm_mx_prepacked with qgemm_prepack_b's layout");
        return mx_common(fmt_a, A, lda_bytes, B, ldb_bytes, scale_a, scale_b, b_layout, bias, C, ldc, M, N, K, stream,
                         false);
    }
    const bool a4 = fmt_a == QGEMM_MX_E2M1;   // e2m1 A with e4m3 B
    if (b_layout != QGEMM_MX_BSCALE_1x32 && b_layout != QGEMM_MX_BSCALE_32x32)
        return fail(QGEMM_ERR_BAD_FORMAT, "unknown B-scale layout %d", (int)b_layout);
    const char *pair = a4 ? "e2m1 x e4m3" : "e4m3 x e2m1";
    const Shape s{M, N, K};
    TRY(check_shape(s, false));
    if (!dma_k_ok(5, K) || (packed && K % 256))
        return fail(QGEMM_ERR_BAD_SHAPE, "K=%lld: %s needs K a multiple of %d", (long long)K, pair,
                    packed ? 256 : 32);
    if (M == 0 || N == 0)
        return QGEMM_OK;
    TRY(check_operand("A", A, lda_bytes, a4 ? K / 2 : K));
    if (packed) {
        // e4m3 B: qgemm_prepack_b's 16-row groups of K-byte rows; e2m1 B:
        // qgemm_prepack_b32's 32-row groups of K/2-byte rows
        if (!B)
            return fail(QGEMM_ERR_NULL_POINTER, "Bp is NULL");
        if (!aligned(B, 16))
            return fail(QGEMM_ERR_BAD_LAYOUT, "Bp is not 16-byte aligned");
    } else {
        TRY(check_operand("B", B, ldb_bytes, a4 ? K : K / 2));
    }
    if (!scale_a)
        return fail(QGEMM_ERR_NULL_POINTER, "scale_a is NULL");
    if (!scale_b)
        return fail(QGEMM_ERR_NULL_POINTER, "scale_b is NULL");
    if (!aligned(scale_a, 8) || !aligned(scale_b, 8))
        return fail(QGEMM_ERR_BAD_LAYOUT, "%s scale arrays must be 8-byte aligned", pair);
    TRY(check_bias(bias));
    TRY(check_output(C, ldc, N, 2));
    TRY(check_device());
    if (a4) {
        const int tile = pick_tile_mx48(s);
        Params p = base_params(A, lda_bytes, B, packed ? K : ldb_bytes, C, ldc, s, K, tile);   // kbytes: B's row
        p.b_packed = packed;
        TRY(check_grid(p));
        p.mx_sa = scale_a;
        p.mx_sb = scale_b;
        p.bias = bias;
        return launch([&] { return launch_mx48(tile, bias != nullptr, (int)b_layout, p, (hipStream_t)stream); });
    }
    int tile = pick_tile_mx84(s);
    if (packed && is_skinny_tile(tile))   // the small-M kernel reads the row-major B only
        tile = DMA128_TILE;
    Params p = base_params(A, lda_bytes, B, packed ? K / 2 : ldb_bytes, C, ldc, s, K, tile);   // kbytes: A's row
    p.b_packed = packed;
    TRY(check_grid(p));
    p.mx_sa = scale_a;
    p.mx_sb = scale_b;
    p.bias = bias;
    return launch([&] { return launch_mx84(tile, bias != nullptr, (int)b_layout, p, (hipStream_t)stream); });
}

qgemm_status qgemm_mx_mixed(qgemm_mx_fmt fmt_a, qgemm_mx_fmt fmt_b, const void *A, int64_t lda_bytes, const void *B,
                            int64_t ldb_bytes, const uint8_t *scale_a, const uint8_t *scale_b,
                            qgemm_mx_bscale b_layout, const uint16_t *bias, uint16_t *C, int64_t ldc, int64_t M,
                            int64_t N, int64_t K, void *stream)
{
    return mx_mixed_common(fmt_a, fmt_b, A, lda_bytes, B, ldb_bytes, scale_a, scale_b, b_layout, bias, C, ldc, M, N, K,
                           stream, false);
}

qgemm_status qgemm_mx_mixed_prepacked(qgemm_mx_fmt fmt_a, qgemm_mx_fmt fmt_b, const void *A, int64_t lda_bytes,
                                      const void *Bp, const uint8_t *scale_a, const uint8_t *scale_b,
                                      qgemm_mx_bscale b_layout, const uint16_t *bias, uint16_t *C, int64_t ldc,
                                      int64_t M, int64_t N, int64_t K, void *stream)
{
    return mx_mixed_common(fmt_a, fmt_b, A, lda_bytes, Bp, 0, scale_a, scale_b, b_layout, bias, C, ldc, M, N, K,
                           stream, true);
}

int64_t qgemm_prepacked_b32_bytes(int64_t N, int64_t row_bytes)
{
    if (N < 0 || row_bytes <= 0 || row_bytes % 128 || N >= LD_LIMIT || row_bytes * 256 >= LD_LIMIT)
        return -1;
    return (N + 31) / 32 * 32 * row_bytes;
}

qgemm_status qgemm_prepack_b32(const void *B, int64_t ldb, int64_t N, int64_t row_bytes, void *Bp, void *stream)
{
    if (N < 0 || N >= LD_LIMIT)
        return fail(QGEMM_ERR_BAD_SHAPE, "N=%lld: need 0 <= N < 2^31", (long long)N);
    if (row_bytes <= 0 || row_bytes % 128 || row_bytes * 256 >= LD_LIMIT)
        return fail(QGEMM_ERR_BAD_SHAPE, "row_bytes=%lld: need a positive multiple of 128, 256 rows below 2^31",
                    (long long)row_bytes);
    if (N == 0)
        return QGEMM_OK;
    TRY(check_operand("B", B, ldb, row_bytes));
    if (!Bp)
        return fail(QGEMM_ERR_NULL_POINTER, "Bp is NULL");
    if (!aligned(Bp, 16))
        return fail(QGEMM_ERR_BAD_LAYOUT, "Bp is not 16-byte aligned");
    TRY(check_device());
    return launch([&] { return launch_prepack_b32((const uint8_t *)B, ldb, N, row_bytes, (uint8_t *)Bp, (hipStream_t)stream); });
}

qgemm_status qgemm_mx(qgemm_mx_fmt fmt, const void *A, int64_t lda_bytes, const void *B, int64_t ldb_bytes,
                      const uint8_t *scale_a, const uint8_t *scale_b, qgemm_mx_bscale b_layout,
                      const uint16_t *bias, uint16_t *C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                      void *stream)
{
    return mx_common(fmt, A, lda_bytes, B, ldb_bytes, scale_a, scale_b, b_layout, bias, C, ldc, M, N, K, stream,
                     false);
}

// ------------------------------------------------------------ prepacked B

int64_t qgemm_prepacked_b_bytes(int64_t N, int64_t row_bytes)
{
    if (N < 0 || row_bytes <= 0 || row_bytes % 256 || N >= LD_LIMIT || row_bytes * 256 >= LD_LIMIT)
        return -1;
    return (N + 15) / 16 * 16 * row_bytes;
}

qgemm_status qgemm_prepack_b(const void *B, int64_t ldb, int64_t N, int64_t row_bytes, void *Bp, void *stream)
{
    if (N < 0 || N >= LD_LIMIT)
        return fail(QGEMM_ERR_BAD_SHAPE, "N=%lld: need 0 <= N < 2^31", (long long)N);
    if (row_bytes <= 0 || row_bytes % 256 || row_bytes * 256 >= LD_LIMIT)
        return fail(QGEMM_ERR_BAD_SHAPE, "row_bytes=%lld: need a positive multiple of 256, 256 rows below 2^31",
                    (long long)row_bytes);
    if (N == 0)
        return QGEMM_OK;
    TRY(check_operand("B", B, ldb, row_bytes));
    if (!Bp)
        return fail(QGEMM_ERR_NULL_POINTER, "Bp is NULL");
    if (!aligned(Bp, 16))
        return fail(QGEMM_ERR_BAD_LAYOUT, "Bp is not 16-byte aligned");
    TRY(check_device());
    return launch([&] { return launch_prepack_b((const uint8_t *)B, ldb, N, row_bytes, (uint8_t *)Bp, (hipStream_t)stream); });
}

qgemm_status qgemm_i8_rowwise_prepacked(const int8_t *A, int64_t lda, const void *Bp, const float *scale_a,
                                        const float *scale_b, const uint16_t *bias, uint16_t *C, int64_t ldc,
                                        int64_t M, int64_t N, int64_t K, void *stream)
{
    return i8_common(A, lda, Bp, 0, scale_a, scale_b, bias, C, ldc, Shape{M, N, K}, stream, OUT_BF16, true);
}

qgemm_status qgemm_f8_pertoken_prepacked(const uint8_t *A, int64_t lda, const void *Bp, const float *scale_a,
                                         const float *scale_b, const uint16_t *bias, uint16_t *C, int64_t ldc,
                                         int64_t M, int64_t N, int64_t K, void *stream)
{
    return f8_common(A, lda, Bp, 0, scale_a, scale_b, bias, C, ldc, M, N, K, stream, true);
}

qgemm_status qgemm_f8_blockscale_prepacked(const uint8_t *A, int64_t lda, const void *Bp, const float *scale_a,
                                           const float *scale_b, const uint16_t *bias, uint16_t *C, int64_t ldc,
                                           int64_t M, int64_t N, int64_t K, void *stream)
{
    return f8b_common(A, lda, Bp, 0, scale_a, scale_b, bias, C, ldc, M, N, K, stream, true);
}

qgemm_status qgemm_mx_prepacked(qgemm_mx_fmt fmt, const void *A, int64_t lda_bytes, const void *Bp,
                                const uint8_t *scale_a, const uint8_t *scale_b, qgemm_mx_bscale b_layout,
                                const uint16_t *bias, uint16_t *C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                                void *stream)
{
    return mx_common(fmt, A, lda_bytes, Bp, 0, scale_a, scale_b, b_layout, bias, C, ldc, M, N, K, stream, true);
}

// ------------------------------------------------------------ quantisers

static qgemm_status check_quant(const uint16_t *X, int64_t ldx, const void *Q, int64_t ldq, int64_t M, int64_t K,
                                int64_t q_row_bytes)
{
    TRY(check_shape(Shape{M, 1, K}, false));
    if (M == 0)
        return QGEMM_OK;
    if (!X)
        return fail(QGEMM_ERR_NULL_POINTER, "X is NULL");
    if (!Q)
        return fail(QGEMM_ERR_NULL_POINTER, "Q is NULL");
    if (!aligned(X, 16) || !aligned(Q, 16))
        return fail(QGEMM_ERR_BAD_LAYOUT, "X and Q must be 16-byte aligned");
    if (ldx < K || ldx % 8 || ldx >= LD_LIMIT)
        return fail(QGEMM_ERR_BAD_LAYOUT, "ldx=%lld elements: need >= K=%lld, a multiple of 8, below 2^31",
                    (long long)ldx, (long long)K);
    if (ldq < q_row_bytes || ldq % 16 || ldq >= LD_LIMIT)
        return fail(QGEMM_ERR_BAD_LAYOUT, "ldq=%lld bytes: need >= %lld, a multiple of 16, below 2^31",
                    (long long)ldq, (long long)q_row_bytes);
    return QGEMM_OK;
}

qgemm_status qgemm_quant_f8_pertoken(const uint16_t *X, int64_t ldx, uint8_t *Q, int64_t ldq, float *scale,
                                     int64_t M, int64_t K, void *stream)
{
    TRY(check_quant(X, ldx, Q, ldq, M, K, K));
    if (M == 0)
        return QGEMM_OK;
    if (!scale)
        return fail(QGEMM_ERR_NULL_POINTER, "scale is NULL");
    if (!aligned(scale, 4))
        return fail(QGEMM_ERR_BAD_LAYOUT, "scale is not 4-byte aligned");
    TRY(check_device());
    return launch([&] { return launch_quant_f8_pertoken(X, ldx, Q, ldq, scale, (int)M, (int)K, (hipStream_t)stream); });
}

qgemm_status qgemm_quant_f8_block(const uint16_t *X, int64_t ldx, uint8_t *Q, int64_t ldq, float *S, int64_t lds,
                                  int64_t M, int64_t K, void *stream)
{
    TRY(check_quant(X, ldx, Q, ldq, M, K, K));
    if (K % 128)
        return fail(QGEMM_ERR_BAD_SHAPE, "K=%lld is not a multiple of 128", (long long)K);
    if (M == 0)
        return QGEMM_OK;
    if (!S)
        return fail(QGEMM_ERR_NULL_POINTER, "S is NULL");
    if (!aligned(S, 4))
        return fail(QGEMM_ERR_BAD_LAYOUT, "S is not 4-byte aligned");
    if (lds < K / 128 || lds >= LD_LIMIT)
        return fail(QGEMM_ERR_BAD_LAYOUT, "lds=%lld elements: need >= K/128=%lld, below 2^31", (long long)lds,
                    (long long)(K / 128));
    TRY(check_device());
    return launch([&] { return launch_quant_f8_block(X, ldx, Q, ldq, S, lds, (int)M, (int)K, (hipStream_t)stream); });
}

qgemm_status qgemm_quant_mx(qgemm_mx_fmt fmt, const uint16_t *X, int64_t ldx, void *Q, int64_t ldq, uint8_t *S,
                            int64_t lds, int64_t M, int64_t K, void *stream)
{
    if (fmt != QGEMM_MX_E4M3 && fmt != QGEMM_MX_E2M1)
        return fail(QGEMM_ERR_BAD_FORMAT, "unknown MX element format %d", (int)fmt);
    TRY(check_quant(X, ldx, Q, ldq, M, K, fmt == QGEMM_MX_E4M3 ? K : K / 2));
    if (M == 0)
        return QGEMM_OK;
    if (!S)
        return fail(QGEMM_ERR_NULL_POINTER, "S is NULL");
    if (lds < K / 32 || lds >= LD_LIMIT)
        return fail(QGEMM_ERR_BAD_LAYOUT, "lds=%lld bytes: need >= K/32=%lld, below 2^31", (long long)lds,
                    (long long)(K / 32));
    TRY(check_device());
    return launch([&] { return launch_quant_mx(fmt == QGEMM_MX_E4M3 ? 0 : 1, X, ldx, (uint8_t *)Q, ldq, S, lds, (int)M, (int)K,
                                  (hipStream_t)stream); });
}

}  // extern "C"
