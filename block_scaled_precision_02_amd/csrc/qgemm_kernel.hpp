// qgemm_kernel.hpp -- gfx950 kernels for the scaled low-precision GEMM
//
//     C[m,n] = bf16( sa[m] * sb[n] * sum_k A[m,k] B[n,k] + bias[n] )
//
// One template covers the three element paths (the rowwise INT8 GEMM of
// comfy-kitchen PR #174 "Optimize HIP WMMA INT8 GEMM staging, epilogue, and
// deep-K tiling"; the per-token FP8 and 32-wide ue8m0 MXFP8 GEMMs of ROCm/mori
// PR #806 "perf(gemm-ar): mxfp8 with row-major scales staged through LDS";
// the MXFP4 GEMM of ROCm/FlyDSL PR #990 "[fp4_gemm_4wave] MXFP4 GEMM perf
// optimize").  Written for CDNA4 only:
//
//  * 256 threads = 4 wave64s in a 2x2 grid; a wave owns a (TM*32) x (TN*32)
//    block of C held in 32x32 MFMA accumulators (TM*TN*16 per lane, so the
//    256x256 tile keeps 256 accumulator registers per lane, which the
//    compiler places in AGPRs).
//  * K advances 128 bytes per step for every element type (128 int8 or e4m3
//    elements, 256 e2m1 elements); each step of A and B is staged HBM ->
//    VGPR -> LDS into one of two LDS buffers, 16-byte chunks XOR-swizzled by
//    row so that the fragment reads of 32 consecutive rows hit distinct banks.
//    Global loads are raw buffer loads whose range check zero-fills rows past
//    M / N; the K tail is zero-filled by pushing its offset out of range in
//    the per-lane VGPR offset (never through soffset, which the range check
//    ignores -- the point made in ROCm/mori PR #806's review thread).
//  * One barrier per K step: step k+1 is written to the idle LDS buffer and
//    step k+2's global loads are issued before the MFMAs of step k start.
//  * MX scales (ue8m0) travel with the operand prefetch straight into VGPRs
//    and feed v_mfma_scale_f32_32x32x64_f8f6f4 as its per-lane scale operand;
//    op_sel picks the byte for each K sub-step.
//  * The MFMA computes C^T (B is the instruction's first operand) so that
//    every lane ends with runs of 4 consecutive n for one m: the epilogue
//    writes 8-byte bf16 vectors.
//  * Epilogue: fixed-order binary32, (float)acc * sa * sb + bias, no
//    contraction (the library is built with -ffp-contract=off), bias add
//    skipped entirely when there is no bias so -0 survives, then RNE to bf16
//    (v_cvt_pk_bf16_f32).  Full tiles store without per-element masks.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace qgemm {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// PATH_F8B: e4m3 with fp32 scales per 128-element K block (A per row, B per
// 128 rows), applied inside the K loop; LDS-fetch kernel only.
// PATH_MX84: MX with e4m3 A and e2m1 B (ue8m0 scales per 32 K elements on
// both); LDS-fetch kernel only.
// PATH_MX6 / PATH_MX6E3: MX with the 6-bit OCP FP6 elements E2M3 / E3M2 (four
// codes per three bytes, lowest bits first); LDS-fetch kernel only.
// PATH_MX48: MX with e2m1 A and e4m3 B (the mixed path with the operands'
// formats the other way round); LDS-fetch kernel only.
// PATH_MX4H: MX e2m1 on both operands in stages of 64 K elements (32-byte
// stage rows, as the mixed paths' e2m1 operand), for K % 128 != 0, where
// PATH_MX4's 64-byte stages would leave part of a stage; LDS-fetch kernel
// only.
enum Path { PATH_I8 = 0, PATH_F8 = 1, PATH_MX8 = 2, PATH_MX4 = 3, PATH_F8B = 4, PATH_MX84 = 5, PATH_MX6 = 6,
            PATH_MX6E3 = 7, PATH_MX48 = 8, PATH_MX4H = 9 };
enum OutKind { OUT_BF16 = 0, OUT_I32 = 1 };

// Kernel arguments (one struct, passed by value).
struct Params {
    const uint8_t *A, *B;          // operand rows, K contiguous
    int64_t lda, ldb;              // row strides in bytes
    const float *scale_a;          // [M] (INT8 / FP8)
    const float *scale_b;          // [N] (INT8 / FP8)
    const uint8_t *mx_sa;          // ue8m0 [M, K/32]      (MX)
    const uint8_t *mx_sb;          // ue8m0 [N or N/32, K/32] (MX)
    const uint16_t *bias;          // [N] bf16 bits or null
    void *C;                       // [M, ldc] bf16 bits (or int32 for OUT_I32)
    int64_t ldc;                   // elements
    int M, N, K;                   // K in elements
    int kbytes;                    // bytes of one operand row
    int ksteps;                    // ceil(kbytes / 128)
    int kblocks;                   // K / 32 (MX scale row length in bytes)
    int tiles_m, tiles_n;
    int group_m;                   // tile rows per group in the launch order
    int b_packed;                  // B in the prepacked layout (LDS-fetch and small-M kernels only):
                                   // 16-row groups of kbytes/64 blocks of 1 KB, B = the group of row 0
    int c_cached;                  // full tiles store C through the caches (else non-temporal)
};

constexpr int KSTEP_BYTES = 128;
constexpr int CHUNKS = KSTEP_BYTES / 16;   // 16-byte chunks per staged row
constexpr unsigned OOB = 0x80000000u;      // offset beyond every range check

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>());
        static_for<I + 1, N>(f);
    }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    // 0x00020000: raw buffer, 32-bit data format, range-checked against bytes.
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 ld16(__amdgpu_buffer_rsrc_t r, unsigned off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// LDS barrier: every LDS write of this wave has landed, then all waves meet.
// Outstanding global loads stay in flight.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The conservative-sync build (QGEMM_SYNC_TWIN=1: libqgemm_sync.so, built
// beside the library for the tests): at every stage boundary of the
// LDS-staged kernels each wave drains all of its outstanding memory and LDS
// operations and the workgroup meets at a barrier.  Its MFMA sequence is the
// fast build's, so the two builds' outputs must be bit-identical; a wait that
// the fast build miscounts (data used before it landed, or overwritten while
// still being read) shows up as a difference.  The small-M kernel takes no
// part: its waves run different numbers of K steps.
#ifndef QGEMM_SYNC_TWIN
#define QGEMM_SYNC_TWIN 0
#endif
__device__ __forceinline__ void twin_sync()
{
    if constexpr (QGEMM_SYNC_TWIN)
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Position of 16-byte chunk c of staged row r inside an LDS tile of rows of
// 128 bytes.  A fragment read has 16 consecutive lanes on 16 consecutive rows
// at the same logical chunk; the slot c ^ f(r), f(r) = (r & 7) ^ ((r >> 3) & 1),
// puts rows r..r+7 in 8 different 16-byte slots of their 128-byte rows and,
// over 16 rows, the even rows and the odd rows each in 8 different slots, so
// neither 8 lanes over 128 bytes of banks nor 16 lanes over 256 bytes collide.
__device__ __forceinline__ int lds_off(int r, int c)
{
    return r * KSTEP_BYTES + ((c ^ (r & 7) ^ ((r >> 3) & 1)) << 4);
}

// Workgroup -> output tile.  Workgroups are handed to the 8 XCDs round-robin;
// renumber so each XCD gets a contiguous run of the grouped order (tiles
// that share A and B panels then share that XCD's L2), then walk the tiles
// in groups of group_m tile rows.  (tile_of_index: the tile of workgroup i.)
__device__ __forceinline__ void tile_of_index(int tiles_m, int tiles_n, int group_m, int i, int &tm, int &tn)
{
    const int G = tiles_m * tiles_n;
    const int xcd = i & 7, local = i >> 3;
    const int per = G >> 3, rem = G & 7;
    const int pid = xcd * per + (xcd < rem ? xcd : rem) + local;
    const int width = group_m * tiles_n;
    const int group = pid / width;
    const int first_m = group * group_m;
    const int gsz = min(tiles_m - first_m, group_m);
    const int in = pid - group * width;
    tm = first_m + in % gsz;
    tn = in / gsz;
}
__device__ __forceinline__ void tile_of(const Params &p, int &tm, int &tn)
{
    tile_of_index(p.tiles_m, p.tiles_n, p.group_m, (int)blockIdx.x, tm, tn);
}

template <int PATH> struct PathTraits;
template <> struct PathTraits<PATH_I8> { static constexpr int NSUB = 4; using Frag = i32x4; };
template <> struct PathTraits<PATH_F8> { static constexpr int NSUB = 2; using Frag = i32x8; };
template <> struct PathTraits<PATH_MX8> { static constexpr int NSUB = 2; using Frag = i32x8; };
template <> struct PathTraits<PATH_MX4> { static constexpr int NSUB = 4; using Frag = i32x8; };
template <> struct PathTraits<PATH_F8B> { static constexpr int NSUB = 2; using Frag = i32x8; };
template <> struct PathTraits<PATH_MX84> { static constexpr int NSUB = 2; using Frag = i32x8; };
template <> struct PathTraits<PATH_MX48> { static constexpr int NSUB = 2; using Frag = i32x8; };
template <> struct PathTraits<PATH_MX4H> { static constexpr int NSUB = 2; using Frag = i32x8; };
template <> struct PathTraits<PATH_MX6> { static constexpr int NSUB = 1; using Frag = i32x8; };
template <> struct PathTraits<PATH_MX6E3> { static constexpr int NSUB = 1; using Frag = i32x8; };

// Fragment of one 32-row MFMA operand for K sub-step S, read from a staged
// tile.  Lane (h = lane/32, row = lane%32):
//   INT8  v_mfma_i32_32x32x32_i8: 16 bytes, chunk 2S+h.
//   e4m3  v_mfma_*_32x32x64_f8f6f4: 32 bytes; the instruction forms its
//         first 32-element K block from VGPRs 0-3 of both lane halves and its
//         second from VGPRs 4-7, so VGPRs 0-3 take chunk 2S+h (block S of the
//         step) and VGPRs 4-7 take chunk 4+2S+h (block 2+S).
//   e2m1  16 bytes = one whole 32-element block per lane: chunk 4h+S (block
//         4h+S of the step's eight); VGPRs 4-7 are unused.
// A and B use the same map, so the products pair up; the scale operand of a
// lane belongs to the block its lane half holds (see scale words below).
template <int PATH, int S>
__device__ __forceinline__ typename PathTraits<PATH>::Frag
load_frag(const uint8_t *tile, int row, int h)
{
    typename PathTraits<PATH>::Frag f;
    if constexpr (PATH == PATH_I8) {
        f = *(const i32x4 *)(tile + lds_off(row, 2 * S + h));
    } else if constexpr (PATH == PATH_MX4) {
        i32x4 lo = *(const i32x4 *)(tile + lds_off(row, 4 * h + S));
        f = i32x8{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
    } else {
        i32x4 lo = *(const i32x4 *)(tile + lds_off(row, 2 * S + h));
        i32x4 hi = *(const i32x4 *)(tile + lds_off(row, 4 + 2 * S + h));
        f = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    return f;
}

template <int PATH> struct AccT { using T = f32x16; };
template <> struct AccT<PATH_I8> { using T = i32x16; };

// acc += B-fragment x A-fragment (the MFMA sees B as its M side: C^T).
template <int PATH, int S>
__device__ __forceinline__ void mfma(typename AccT<PATH>::T &acc,
                                     const typename PathTraits<PATH>::Frag &fb,
                                     const typename PathTraits<PATH>::Frag &fa,
                                     unsigned sc_b, unsigned sc_a)
{
    if constexpr (PATH == PATH_I8) {
        acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb, fa, acc, 0, 0, 0);
    } else if constexpr (PATH == PATH_F8 || PATH == PATH_F8B) {
        // scale operands 0 with op_sel 0: the unscaled f8f6f4 encoding.
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb, fa, acc, 0, 0, 0, 0, 0, 0);
    } else if constexpr (PATH == PATH_MX8) {
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb, fa, acc, 0, 0, S, (int)sc_b, S, (int)sc_a);
    } else if constexpr (PATH == PATH_MX84) {
        // first operand (B) e2m1: cbsz = 4; second (A) e4m3: blgp = 0
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb, fa, acc, 4, 0, S, (int)sc_b, S, (int)sc_a);
    } else if constexpr (PATH == PATH_MX4H) {
        // both operands e2m1: cbsz = blgp = 4
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb, fa, acc, 4, 4, S, (int)sc_b, S, (int)sc_a);
    } else if constexpr (PATH == PATH_MX48) {
        // first operand (B) e4m3: cbsz = 0; second (A) e2m1: blgp = 4
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb, fa, acc, 0, 4, S, (int)sc_b, S, (int)sc_a);
    } else if constexpr (PATH == PATH_MX6) {
        // FP6 E2M3 operands: format code 2 (VGPRs 0-5 of each operand)
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb, fa, acc, 2, 2, S, (int)sc_b, S, (int)sc_a);
    } else if constexpr (PATH == PATH_MX6E3) {
        // FP6 E3M2 operands: format code 3
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb, fa, acc, 3, 3, S, (int)sc_b, S, (int)sc_a);
    } else {
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb, fa, acc, 4, 4, S, (int)sc_b, S, (int)sc_a);
    }
}

// ue8m0 scale word for one lane and one K step.  The lane half h needs the
// blocks its fragments hold in sub-steps 0..NSUB-1, packed so that byte S is
// sub-step S's scale:
//   e2m1: blocks 4h..4h+3 of the step  -> 4 consecutive bytes
//   e4m3: blocks 2h, 2h+1 of the step  -> 2 consecutive bytes
// SVEC: the bytes are read with one aligned load (scale rows are whole
// dwords / halfwords); otherwise byte by byte.  Blocks at or past K/32 read
// as 0 (their data is zero as well).
template <int PATH, bool SVEC>
__device__ __forceinline__ unsigned load_scale_word(__amdgpu_buffer_rsrc_t r, int row_off, int kt,
                                                    int h, int kblocks)
{
    constexpr int NB = (PATH == PATH_MX4) ? 8 : 4;   // blocks per K step
    constexpr int NL = (PATH == PATH_MX4) ? 4 : 2;   // blocks per lane half
    const int b0 = kt * NB + h * NL;
    if constexpr (SVEC) {
        const unsigned off = (b0 < kblocks) ? (unsigned)(row_off + b0) : OOB;
        if constexpr (NL == 4)
            return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
        else
            return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
    } else {
        unsigned w = 0;
#pragma unroll
        for (int q = 0; q < NL; ++q) {
            const unsigned off = (b0 + q < kblocks) ? (unsigned)(row_off + b0 + q) : OOB;
            w |= (unsigned)__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0) << (8 * q);
        }
        return w;
    }
}

__device__ __forceinline__ unsigned pack_bf16(float x, float y)
{
    bf16x2 v;
    v[0] = (__bf16)x;
    v[1] = (__bf16)y;
    return __builtin_bit_cast(unsigned, v);
}

// ------------------------------------------------------------ epilogue
// Per-tile epilogue operands (row scales, column scales, bias) parked in LDS
// while the K loop runs, so the epilogue reads them at LDS latency instead of
// waiting on memory between groups of outputs:
//   [0, 1024)     scale_a[m0 .. m0+BM) fp32
//   [1024, 2048)  scale_b[n0 .. n0+BN) fp32
//   [2048, 2560)  bias[n0 .. n0+BN) bf16; [2560, 3072) absorbs a 16-byte-per-
//                 lane fetch's unused half
// Only full tiles read them; an edge tile loads element by element.
constexpr int PRM_SB = 1024, PRM_BIAS = 2048, PRM_BYTES = 3072;

// Cache policy of the whole-row output stores: non-temporal.  C is written
// once and never read back by the kernel; streaming it past the caches leaves
// L2 to the A and B panels that neighbouring tiles share (one MI355X: INT8
// 30000x21504x5376 +3%, MXFP4 8192^3 +3%, MXFP8 16384x7168x2048 +9%).  Stores
// of partial rows (edge tiles) keep the default policy: written past the
// caches, partial lines cost far more.
constexpr int CPOL_NT = 2;

constexpr int pow2_at_least(int x) { return x <= 1 ? 1 : 2 * pow2_at_least((x + 1) / 2); }

// Shared by the kernels: scale, bias, round and store one workgroup tile.
// LDSBYTES is the LDS at lds_base the kernel owns (reused as the output
// stash once every wave is done with the operand buffers); prm is the
// parked epilogue operands (used by full tiles when PRM).
template <int PATH, int WM, int WN, int TM, int TN, bool BIAS, int OUT, int LDSBYTES, bool PRM, class Acc>
__device__ __forceinline__ void store_tile(const Params &p, Acc (&acc)[TM][TN], uint8_t *lds_base,
                                           const uint8_t *prm, int m0, int n0, int rows_a, int rows_b)
{
    constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
    // MX and blockscale apply their scales inside the K loop: the epilogue
    // only adds the bias and rounds
    constexpr bool MX = (PATH == PATH_MX8 || PATH == PATH_MX4 || PATH == PATH_F8B || PATH == PATH_MX84 ||
                         PATH == PATH_MX48 || PATH == PATH_MX4H || PATH == PATH_MX6 || PATH == PATH_MX6E3);
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int h = lane >> 5, r32 = lane & 31;
    const int arow = wm * TM * 32 + r32;
    // Lane holds, for tile (i, j): m = m0 + arow + 32i, and for g = 0..3 the
    // four consecutive n = n0 + wn*TN*32 + 32j + 8g + 4h + {0..3} in
    // acc[i][j][4g..4g+3].  Every global access goes through a range-checked
    // buffer descriptor: loads past M / N read 0, stores past them are
    // dropped, so the only difference between a full tile and an edge tile
    // is that the edge tile loads its operands and stores its results element
    // by element (columns past N inside a row of ldc must not be touched).
    constexpr int ESZ = (OUT == OUT_I32) ? 4 : 2;
    const bool full = (rows_a == BM) && (rows_b == BN);
    const int nloc_base = wn * TN * 32 + 4 * h;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc((const uint8_t *)p.C + (int64_t)m0 * p.ldc * ESZ,
                                                (uint32_t)((int64_t)rows_a * p.ldc * ESZ));
    const unsigned col0 = (unsigned)(n0 * ESZ);
    __amdgpu_buffer_rsrc_t rsb_e, rbias;
    if constexpr (OUT == OUT_BF16 && !MX)
        rsb_e = make_rsrc(p.scale_b + n0, (uint32_t)(rows_b * 4));
    if constexpr (BIAS)
        rbias = make_rsrc(p.bias + n0, (uint32_t)(rows_b * 2));
    // Full bf16 tiles leave through LDS: each wave parks its (TM*32) x (TN*32)
    // block of bf16 results in its own stash (16-byte chunks XOR-swizzled by
    // row), then writes whole 16-byte row pieces, consecutive lanes covering
    // consecutive bytes of a row, so every store instruction fills complete
    // cache lines instead of touching 32 rows.  A stash row holds the wave's
    // SCHK chunks in PCHK slots (the next power of two: 192-byte rows of the
    // 192x192 tile take 256).
    constexpr int SCHK = TN * 32 * 2 / 16;          // 16-byte chunks of a wave's row (bf16)
    constexpr int PCHK = pow2_at_least(SCHK);       // stash slots per row
    constexpr int SPITCH = PCHK * 16;               // stash row pitch
    constexpr bool STASH = OUT == OUT_BF16 && PCHK <= 64 && WM * WN * TM * 32 * SPITCH <= LDSBYTES;
    uint8_t *stash = lds_base + wave * (TM * 32) * SPITCH;
    if constexpr (STASH) {
        if (full)
            lds_barrier();   // every wave is done with the operand buffers
    }
    // Full tiles and edge tiles each get straight-line code.
    auto body = [&](auto fullc) {
        constexpr bool FULL = decltype(fullc)::value;
        // Row scales of the lane's TM rows.
        float sa[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            sa[i] = 0.f;
            if constexpr (OUT == OUT_BF16 && !MX) {
                const int mloc = arow + 32 * i;
                if (PRM && FULL)
                    sa[i] = *(const float *)(prm + 4 * mloc);
                else if (mloc < rows_a)
                    sa[i] = p.scale_a[m0 + mloc];
            }
        }
        // Column groups outermost: a group's scales and bias serve all TM rows.
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int nloc = nloc_base + 32 * j + 8 * g;
                unsigned sbw[4] = {0, 0, 0, 0}, bbw[4] = {0, 0, 0, 0};
                if constexpr (OUT == OUT_BF16) {
                    // Per-column scale and bias: parked copies or one vector load
                    // in a full tile; element loads at an edge (a vector load that
                    // runs past the range returns zeros for all of its elements).
                    if constexpr (FULL) {
                        if constexpr (!MX) {
                            const u32x4 t = PRM ? *(const u32x4 *)(prm + PRM_SB + 4 * nloc)
                                                : ld16(rsb_e, (unsigned)(nloc * 4));
#pragma unroll
                            for (int r = 0; r < 4; ++r) sbw[r] = t[r];
                        }
                        if constexpr (BIAS) {
                            const u32x2 t = PRM ? *(const u32x2 *)(prm + PRM_BIAS + 2 * nloc)
                                                : __builtin_amdgcn_raw_buffer_load_b64(rbias, (unsigned)(nloc * 2), 0, 0);
                            const unsigned t0 = t[0], t1 = t[1];
                            bbw[0] = t0 << 16;
                            bbw[1] = t0 & 0xffff0000u;
                            bbw[2] = t1 << 16;
                            bbw[3] = t1 & 0xffff0000u;
                        }
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const bool in = nloc + r < rows_b;
                            if constexpr (!MX)
                                sbw[r] = __builtin_amdgcn_raw_buffer_load_b32(
                                    rsb_e, in ? (unsigned)((nloc + r) * 4) : OOB, 0, 0);
                            if constexpr (BIAS)
                                bbw[r] = (unsigned)__builtin_amdgcn_raw_buffer_load_b16(
                                             rbias, in ? (unsigned)((nloc + r) * 2) : OOB, 0, 0) << 16;
                        }
                    }
                }
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const int mloc = arow + 32 * i;
                    const unsigned off = (unsigned)((int64_t)mloc * p.ldc * ESZ) + col0 + (unsigned)(nloc * ESZ);
                    if constexpr (OUT == OUT_I32) {
                        const i32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1],
                                         acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                        if constexpr (FULL) {
                            if (p.c_cached)
                                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rc, off, 0, 0);
                            else
                                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rc, off, 0,
                                                                       CPOL_NT);
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                __builtin_amdgcn_raw_buffer_store_b32(
                                    (unsigned)v[r], rc, (nloc + r < rows_b) ? off + 4 * r : OOB, 0, 0);
                        }
                    } else {
                        float f[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            float x;
                            if constexpr (PATH == PATH_I8)
                                x = (float)acc[i][j][4 * g + r];
                            else
                                x = acc[i][j][4 * g + r];
                            // (scalars only under bit_cast: clang's bit_cast of an
                            // ext_vector element reads element 0)
                            if constexpr (!MX) {
                                x = x * sa[i];
                                x = x * __builtin_bit_cast(float, sbw[r]);
                            }
                            if constexpr (BIAS)
                                x = x + __builtin_bit_cast(float, bbw[r]);
                            f[r] = x;
                        }
                        const u32x2 v = {pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3])};
                        if constexpr (FULL && !STASH) {
                            __builtin_amdgcn_raw_buffer_store_b64(v, rc, off, 0, 0);
                        } else if constexpr (FULL) {
                            // park in this wave's LDS stash (written out below)
                            const int srow = 32 * i + r32;
                            const int chunk = 4 * j + g;
                            *(u32x2 *)(stash + srow * SPITCH + ((chunk ^ (srow & (PCHK - 1))) << 4) + 8 * h) = v;
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                __builtin_amdgcn_raw_buffer_store_b16(
                                    (unsigned short)(v[r >> 1] >> (16 * (r & 1))), rc,
                                    (nloc + r < rows_b) ? off + 2 * r : OOB, 0, 0);
                        }
                    }
                }
            }
        }
    };
    if (full)
        body(std::true_type());
    else
        body(std::false_type());
    if constexpr (STASH) {
        if (full) {
            constexpr int LPR = PCHK;                   // lanes per stash row (those past SCHK idle)
            constexpr int RPI = 64 / LPR;               // rows per store instruction
            const int c = lane % LPR;
            const unsigned gbase = (unsigned)((int64_t)(wm * TM * 32) * p.ldc * 2) + col0 +
                                   (unsigned)((wn * TN * 32) * 2 + c * 16);
#pragma unroll
            for (int it = 0; it < TM * 32 / RPI; ++it) {
                const int srow = it * RPI + lane / LPR;
                const u32x4 v = *(const u32x4 *)(stash + srow * SPITCH + ((c ^ (srow & (PCHK - 1))) << 4));
                const unsigned off = c < SCHK ? gbase + (unsigned)(srow * p.ldc * 2) : OOB;
                if (p.c_cached)
                    __builtin_amdgcn_raw_buffer_store_b128(v, rc, off, 0, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b128(v, rc, off, 0, CPOL_NT);
            }
        }
    }
}

template <int PATH, int WM, int WN, int TM, int TN, bool BIAS, int BROWS, bool SVEC, int OUT>
__global__ void __launch_bounds__(64 * WM * WN, 1) qgemm_kernel(const Params p)
{
    constexpr int NT = 64 * WM * WN;        // threads: WM x WN waves
    constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
    constexpr int RSTEP = NT / CHUNKS;      // rows staged per pass of the workgroup
    constexpr int NSUB = PathTraits<PATH>::NSUB;
    constexpr int CA = BM * CHUNKS / NT;    // A chunks staged per thread per step
    constexpr int CB = BN * CHUNKS / NT;
    static_assert(CA * NT == BM * CHUNKS && CB * NT == BN * CHUNKS, "tile / thread mismatch");
    constexpr bool MX = (PATH == PATH_MX8 || PATH == PATH_MX4);
    using Frag = typename PathTraits<PATH>::Frag;
    using Acc = typename AccT<PATH>::T;

    __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + BN) * KSTEP_BYTES];
    constexpr bool PRM = OUT == OUT_BF16 && (!MX || BIAS);
    __shared__ __attribute__((aligned(16))) uint8_t prm[PRM ? PRM_BYTES : 16];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int h = lane >> 5, r32 = lane & 31;

    int tm, tn;
    tile_of(p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int rows_a = min(BM, p.M - m0), rows_b = min(BN, p.N - n0);

    // Operand ranges: rows past M / N and everything after the last valid
    // row's K bytes are out of range and read as zero.
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A + (int64_t)m0 * p.lda,
                                                (uint32_t)((rows_a - 1) * p.lda + p.kbytes));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B + (int64_t)n0 * p.ldb,
                                                (uint32_t)((rows_b - 1) * p.ldb + p.kbytes));

    // Staging map: thread tid copies chunk tid%8 of rows tid/8 + RSTEP*i.
    // RS register sets: step s is fetched into set s%RS, parked in LDS buffer
    // s&1 during step s-1, and its set is then refilled with step s+RS.  Two
    // sets (fetch ~1.75 steps ahead) where the fragments are 16 bytes; one
    // set (~0.75 steps) for e4m3, whose 32-byte fragments leave no room.
    constexpr int RS = (PATH == PATH_F8 || PATH == PATH_MX8) ? 1 : 2;
    const int st_row = tid >> 3, st_c = tid & 7;
    u32x4 ga[RS][CA], gb[RS][CB];

    // MX scale ranges and per-lane row offsets.
    __amdgpu_buffer_rsrc_t rsa, rsb;
    int sa_off[TM], sb_off[TN];
    unsigned sa_ld[RS][TM], sb_ld[RS][TN];
    if constexpr (MX) {
        rsa = make_rsrc(p.mx_sa + (int64_t)m0 * p.kblocks, (uint32_t)(rows_a * p.kblocks));
        if constexpr (BROWS == 1) {
            rsb = make_rsrc(p.mx_sb + (int64_t)n0 * p.kblocks, (uint32_t)(rows_b * p.kblocks));
        } else {
            rsb = make_rsrc(p.mx_sb + (int64_t)(n0 / 32) * p.kblocks,
                            (uint32_t)(((rows_b + 31) / 32) * p.kblocks));
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
            sa_off[i] = (wm * TM * 32 + i * 32 + r32) * p.kblocks;
#pragma unroll
        for (int j = 0; j < TN; ++j)
            sb_off[j] = (BROWS == 1 ? (wn * TN * 32 + j * 32 + r32) : (wn * TN + j)) * p.kblocks;
    }

    auto load_step = [&](int kt, auto setc) {
        constexpr int SET = decltype(setc)::value;
        const int kb = kt * KSTEP_BYTES + st_c * 16;
        const bool kin = kb < p.kbytes;
#pragma unroll
        for (int i = 0; i < CA; ++i)
            ga[SET][i] = ld16(ra, kin ? (unsigned)((st_row + RSTEP * i) * p.lda + kb) : OOB);
#pragma unroll
        for (int i = 0; i < CB; ++i)
            gb[SET][i] = ld16(rb, kin ? (unsigned)((st_row + RSTEP * i) * p.ldb + kb) : OOB);
        if constexpr (MX) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
                sa_ld[SET][i] = load_scale_word<PATH, SVEC>(rsa, sa_off[i], kt, h, p.kblocks);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                sb_ld[SET][j] = load_scale_word<PATH, SVEC>(rsb, sb_off[j], kt, h, p.kblocks);
        }
    };
    auto store_step = [&](int buf, auto setc) {
        constexpr int SET = decltype(setc)::value;
        uint8_t *ta = &lds[buf][0];
        uint8_t *tb = &lds[buf][BM * KSTEP_BYTES];
#pragma unroll
        for (int i = 0; i < CA; ++i)
            *(u32x4 *)(ta + lds_off(st_row + RSTEP * i, st_c)) = ga[SET][i];
#pragma unroll
        for (int i = 0; i < CB; ++i)
            *(u32x4 *)(tb + lds_off(st_row + RSTEP * i, st_c)) = gb[SET][i];
    };

    Acc acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = Acc{};

    const int arow = wm * TM * 32 + r32;
    const int brow = wn * TN * 32 + r32;

    // Fragments of two consecutive K sub-steps (S even -> set 0, odd -> 1).
    Frag fa[2][TM], fb[2][TN];
    // MX scale words of the step being multiplied and of the step parked next.
    unsigned sa_use[TM], sb_use[TN], sa_nxt[TM], sb_nxt[TN];

    auto read_frags = [&](auto sc, int buf, auto setc) {
        constexpr int S = decltype(sc)::value;
        constexpr int SET = decltype(setc)::value;
        const uint8_t *ta = &lds[buf][0];
        const uint8_t *tb = &lds[buf][BM * KSTEP_BYTES];
#pragma unroll
        for (int i = 0; i < TM; ++i)
            fa[SET][i] = load_frag<PATH, S>(ta, arow + 32 * i, h);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            fb[SET][j] = load_frag<PATH, S>(tb, brow + 32 * j, h);
    };
    // MFMAs of sub-step S over tile pairs [Q0, Q1) of the TM*TN grid, in
    // serpentine order (consecutive MFMAs share a fragment).
    auto mfmas = [&](auto sc, auto q0c, auto q1c) {
        constexpr int S = decltype(sc)::value;
        constexpr int SET = S & 1;
        static_for<decltype(q0c)::value, decltype(q1c)::value>([&](auto qc) {
            constexpr int Q = decltype(qc)::value;
            constexpr int i = Q / TN;
            constexpr int j = (i & 1) ? (TN - 1 - Q % TN) : (Q % TN);
            mfma<PATH, S>(acc[i][j], fb[SET][j], fa[SET][i], MX ? sb_use[j] : 0u, MX ? sa_use[i] : 0u);
        });
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    // Prologue: the tile's epilogue operands (one per thread, ahead of the
    // operand loads), steps 0..RS-1 into the register sets, step 0 into LDS
    // buffer 0, step RS into set 0, then the sub-step 0 fragments of step 0.
    unsigned pv_sa = 0, pv_sb = 0;
    unsigned short pv_bias = 0;
    if constexpr (PRM) {
        if (tid < BM) {
            if constexpr (!MX) {
                const __amdgpu_buffer_rsrc_t r = make_rsrc(p.scale_a + m0, (uint32_t)(rows_a * 4));
                pv_sa = __builtin_amdgcn_raw_buffer_load_b32(r, tid < rows_a ? (unsigned)(4 * tid) : OOB, 0, 0);
            }
        }
        if (tid < BN) {
            if constexpr (!MX) {
                const __amdgpu_buffer_rsrc_t r = make_rsrc(p.scale_b + n0, (uint32_t)(rows_b * 4));
                pv_sb = __builtin_amdgcn_raw_buffer_load_b32(r, tid < rows_b ? (unsigned)(4 * tid) : OOB, 0, 0);
            }
            if constexpr (BIAS) {
                const __amdgpu_buffer_rsrc_t r = make_rsrc(p.bias + n0, (uint32_t)(rows_b * 2));
                pv_bias = __builtin_amdgcn_raw_buffer_load_b16(r, tid < rows_b ? (unsigned)(2 * tid) : OOB, 0, 0);
            }
        }
    }
    load_step(0, I0());
    if constexpr (RS == 2)
        load_step(1, I1());
    store_step(0, I0());
    if constexpr (MX) {
#pragma unroll
        for (int i = 0; i < TM; ++i) sa_use[i] = sa_ld[0][i];
#pragma unroll
        for (int j = 0; j < TN; ++j) sb_use[j] = sb_ld[0][j];
    }
    load_step(RS, I0());
    if constexpr (PRM) {
        if (tid < BM && !MX)
            *(unsigned *)(prm + 4 * tid) = pv_sa;
        if (tid < BN) {
            if constexpr (!MX)
                *(unsigned *)(prm + PRM_SB + 4 * tid) = pv_sb;
            if constexpr (BIAS)
                *(unsigned short *)(prm + PRM_BIAS + 2 * tid) = pv_bias;
        }
    }
    lds_barrier();
    read_frags(I0(), 0, I0());

    // One K step.  Region A (before the barrier): park step kt+1 (register
    // set (kt+1)&1) in the idle LDS buffer -- it was last read before the
    // previous barrier -- refill that set with step kt+3, and read the
    // fragments of sub-steps 1..NSUB-1 while the MFMAs of the sub-step before
    // run.  Half-way through the last sub-step every wave has finished
    // reading buffer cur and its LDS writes have landed: barrier.  Region B:
    // the sub-step 0 fragments of step kt+1 come from the other buffer under
    // the last MFMAs.
    constexpr int NQ = TM * TN;
    constexpr int RPF = (PATH == PATH_F8 || PATH == PATH_MX8) ? 2 : 1;   // ds_reads per fragment
    constexpr int NDSR = (TM + TN) * RPF;                               // per sub-step
    constexpr int NSTG = CA + CB;                                       // staged chunks per thread
    constexpr int NSCL = MX ? (TM + TN) * (SVEC ? 1 : (PATH == PATH_MX4 ? 4 : 2)) : 0;
    auto kstep = [&](int kt, auto setc0, auto storec, auto loadc, auto nextc) {
        constexpr int SET = decltype(setc0)::value % RS;   // register set of step kt+1
        using setc = std::integral_constant<int, SET>;
        constexpr bool STORE = decltype(storec)::value;
        constexpr bool LOAD = decltype(loadc)::value;
        constexpr bool NEXT = decltype(nextc)::value;
        const int cur = kt & 1;
        static_for<0, NSUB>([&](auto sc) {
            constexpr int S = decltype(sc)::value;
            if constexpr (S == 0 && STORE) {
                store_step(cur ^ 1, setc());
                if constexpr (MX) {
#pragma unroll
                    for (int i = 0; i < TM; ++i) sa_nxt[i] = sa_ld[SET][i];
#pragma unroll
                    for (int j = 0; j < TN; ++j) sb_nxt[j] = sb_ld[SET][j];
                }
            }
            if constexpr (S == 1 && LOAD)
                load_step(kt + 1 + RS, setc());
            if constexpr (S + 1 < NSUB)
                read_frags(std::integral_constant<int, S + 1>(), cur, std::integral_constant<int, (S + 1) & 1>());
            if constexpr (S + 1 < NSUB) {
                mfmas(sc, I0(), std::integral_constant<int, NQ>());
            } else {
                mfmas(sc, I0(), std::integral_constant<int, NQ / 2>());
            }
        });
        // Issue order for region A: each MFMA followed by its share of the
        // sub-step's memory operations.
        static_for<0, NSUB>([&](auto sc) {
            constexpr int S = decltype(sc)::value;
            constexpr int NM = (S + 1 < NSUB) ? NQ : NQ / 2;
            constexpr int W = (S == 0 && STORE) ? NSTG : 0;
            constexpr int V = (S == 1 && LOAD) ? NSTG + NSCL : 0;
            constexpr int R = (S + 1 < NSUB) ? NDSR : 0;
            static_for<0, NM>([&](auto jc) {
                constexpr int J = decltype(jc)::value;
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                constexpr int w = W * (J + 1) / NM - W * J / NM;
                constexpr int v = V * (J + 1) / NM - V * J / NM;
                constexpr int r = R * (J + 1) / NM - R * J / NM;
                if constexpr (w > 0) __builtin_amdgcn_sched_group_barrier(0x200, w, 0);
                if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x020, v, 0);
                if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
            });
        });
        if constexpr (NEXT) {
            __builtin_amdgcn_sched_barrier(0);
            twin_sync();
            lds_barrier();
            __builtin_amdgcn_sched_barrier(0);
            read_frags(I0(), cur ^ 1, I0());
        }
        mfmas(std::integral_constant<int, NSUB - 1>(), std::integral_constant<int, NQ / 2>(),
              std::integral_constant<int, NQ>());
        if constexpr (NEXT) {
            static_for<0, NQ / 2>([&](auto jc) {
                constexpr int J = decltype(jc)::value;
                constexpr int NM = NQ / 2;
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                constexpr int r = NDSR * (J + 1) / NM - NDSR * J / NM;
                if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
            });
            if constexpr (MX) {
#pragma unroll
                for (int i = 0; i < TM; ++i) sa_use[i] = sa_nxt[i];
#pragma unroll
                for (int j = 0; j < TN; ++j) sb_use[j] = sb_nxt[j];
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        twin_sync();
        __builtin_amdgcn_sched_barrier(0);
    };

    // Steps alternate register sets, so the loop handles two at a time.  The
    // step count is rounded up to even: fetches past K read zeros (the K
    // predicate pushes them out of range, scale words included), so a step
    // past the end adds exact zeros to the accumulators, and the loads and
    // parks of steps beyond it touch no memory that is read back.
    const int ks2 = (p.ksteps + 1) & ~1;
    for (int kt = 0; kt < ks2; kt += 2) {
        kstep(kt, I1(), std::true_type(), std::true_type(), std::true_type());
        kstep(kt + 1, I0(), std::true_type(), std::true_type(), std::true_type());
    }

    store_tile<PATH, WM, WN, TM, TN, BIAS, OUT, 2 * (BM + BN) * KSTEP_BYTES, PRM>(p, acc, &lds[0][0], prm, m0, n0,
                                                                           rows_a, rows_b);
}

}  // namespace qgemm
