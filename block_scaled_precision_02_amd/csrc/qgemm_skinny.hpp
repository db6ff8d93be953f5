// qgemm_skinny.hpp -- the scaled GEMM for small M, where the call is bound by
// streaming B from HBM rather than by the matrix cores.
//
//     C[m,n] = bf16( sa[m] * sb[n] * sum_k A[m,k] B[n,k] + bias[n] )   (INT8, FP8)
//     C[m,n] = bf16( sum_k A~[m,k] B~[n,k] + bias[n] )                  (MX)
//
// The 256x256 tiles of the main kernels leave most CUs idle when M is a few
// rows (a 2112-column B gives 9 tiles of 256): here a workgroup owns 16
// columns of C (one 16x16 MFMA block wide) and TM blocks of 16 rows, and
// its eight waves split K: wave w takes the K steps w, w+8, w+16, ...
// (2112 columns -> 132 workgroups, each streaming 16 rows of B with eight
// waves in flight).  The partial sums meet in LDS and are added in wave
// order, so the result does not depend on timing.
//
//  * No LDS staging: a 16x16 MFMA operand is 16 rows with four lanes per row,
//    so a wave's 16-byte-per-lane load of one operand fragment reads 16 rows
//    x 64 contiguous bytes -- the same row pieces the LDS-fetch kernels use.
//    The sum over K does not depend on which K a lane holds as long as A and
//    B agree, so lane group g (lane / 16) takes byte chunk g of each 64-byte
//    piece (and, for the 128-byte e4m3 step, chunk g + 4 in its upper half).
//  * Each wave keeps D steps of fragments in flight in a register ring (the
//    compiler waits on each slot's loads just before its MFMA).
//  * Rows past M / N read zeros through the buffer range check (their offset
//    is pushed out of range, and stays out of range after any K offset);
//    16-byte chunks at or past the row's K bytes read zeros the same way, so
//    K needs no multiple beyond the 32 every call has.
//  * Output: with B as the instruction's first operand each lane ends with
//    four consecutive n for one m (lane l: m = 16i + l%16, n = 4(l/16) + r),
//    stored as one 8-byte vector when the four columns exist.
//  * MX (v_mfma_scale_f32_16x16x128_f8f6f4 with ue8m0 scale operands): a
//    step is 128 elements, four 32-element blocks, and lane group g gives the
//    scale of block g of the step (the instruction applies a lane group's
//    scale to the block that the same group position holds in its own K
//    order: for e4m3, VGPRs 0-3 of groups 2j, 2j+1 form block j < 2 and VGPRs
//    4-7 form blocks 2 and 3, which the map above -- chunks g and g + 4 --
//    makes the step's blocks in K order; for e2m1 a group's 16 bytes are its
//    block).  Scale bytes are loaded per lane and step; blocks past K/32 and
//    rows past M / N read 0, whose data is zero too.
//  * Mixed MX (e4m3 A, e2m1 B): A keeps the e4m3 map (chunks g and g + 4 of a
//    128-byte step); a step of B is 64 bytes, lane group g's 16 bytes being
//    block g -- the block the same lane group's e4m3 chunks form -- and the
//    instruction takes B as FP4 (cbsz 4) and A as FP8.
//  * FP8 blockscale (fp32 scales per 128-element K block): a step is exactly
//    one block, so each step's MFMA starts a fresh partial sum and the lane
//    folds it into its total with fma(partial, sa[m, s] * sb[n/128, s]); the
//    16 columns of a workgroup lie in one 128-row group of B.
#pragma once
#include "qgemm_kernel.hpp"

namespace qgemm {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int PATH> struct SkinnyTraits;
// K bytes per MFMA step; 16-byte chunks per lane per step
template <> struct SkinnyTraits<PATH_I8> {
    static constexpr int KSTEP = 64, NCH = 1;
    using Frag = i32x4;
    using Acc = i32x4;
};
template <> struct SkinnyTraits<PATH_F8> {
    static constexpr int KSTEP = 128, NCH = 2;
    using Frag = i32x8;
    using Acc = f32x4;
};
template <> struct SkinnyTraits<PATH_MX8> {
    static constexpr int KSTEP = 128, NCH = 2;
    using Frag = i32x8;
    using Acc = f32x4;
};
template <> struct SkinnyTraits<PATH_MX4> {   // 64 bytes = 128 e2m1 elements
    static constexpr int KSTEP = 64, NCH = 1;
    using Frag = i32x4;                       // the low half of the instruction's operand
    using Acc = f32x4;
};
template <> struct SkinnyTraits<PATH_MX84> {  // A: 128 e4m3 bytes; B: 64 e2m1 bytes (its low half)
    static constexpr int KSTEP = 128, NCH = 2;
    using Frag = i32x8;
    using Acc = f32x4;
};
template <> struct SkinnyTraits<PATH_F8B> {
    static constexpr int KSTEP = 128, NCH = 2;
    using Frag = i32x8;
    using Acc = f32x4;
};

constexpr int SK_WAVES = 8;

// Steps in flight per wave: the register ring is D x (TM + 1) fragments (and,
// for MX, as many scale bytes) and a wave has 256 registers at two waves per
// SIMD.  The 16-row MX forms keep to 128 registers so that two workgroups
// share a CU: an MX weight's K is often short (2048 e4m3 = 16 steps, 2 per
// wave), so a workgroup's time is mostly one memory round trip, and 7168
// columns make 448 workgroups -- one round with two per CU instead of two
// (MXFP8 1 x 7168 x 2048: 13.2 -> 8.0 us).
template <int PATH, int TM> constexpr int skinny_depth()
{
    if constexpr (PATH == PATH_MX4)
        return TM == 1 ? 8 : 4;
    if constexpr (PATH == PATH_MX8 || PATH == PATH_MX84 || PATH == PATH_F8B)
        return TM == 1 ? 4 : 2;
    return TM == 1 ? (PATH == PATH_I8 ? 16 : 8) : (PATH == PATH_I8 ? 8 : 4);
}

template <int PATH, int TM, int D, bool BIAS, int BROWS>
__global__ void __launch_bounds__(64 * SK_WAVES,
                                  ((PATH == PATH_MX8 || PATH == PATH_MX4 || PATH == PATH_MX84 || PATH == PATH_F8B) &&
                                   TM == 1) ? 2 : 1)
    qgemm_skinny_kernel(const Params p)
{
    using T = SkinnyTraits<PATH>;
    using Frag = typename T::Frag;
    using Acc = typename T::Acc;
    constexpr bool MX = PATH == PATH_MX8 || PATH == PATH_MX4 || PATH == PATH_MX84;
    constexpr bool B4 = PATH == PATH_MX84;          // e2m1 B under e4m3 A: 64 B of B per step
    constexpr bool BS = PATH == PATH_F8B;           // fp32 scales per 128-element K block
    constexpr bool INK = MX || BS;                  // scales applied inside the K loop
    constexpr int BM = 16 * TM, BN = 16;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, g = lane >> 4;

    int tm, tn;
    tile_of(p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int rows_a = min(BM, p.M - m0), rows_b = min(BN, p.N - n0);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A + (int64_t)m0 * p.lda,
                                                (uint32_t)((rows_a - 1) * p.lda + p.kbytes));
    // B row-major, or prepacked (the workgroup's 16 columns are one packed
    // group: 64-byte K piece t of its rows is the 1 KB block t, row r's chunk
    // c at slot 4r + (c ^ ((r >> 2) & 3)); rows past N are zeros there)
    const int kbytes_b = B4 ? p.kbytes / 2 : p.kbytes;
    const __amdgpu_buffer_rsrc_t rb =
        p.b_packed ? make_rsrc(p.B + (int64_t)(n0 / 16) * 16 * p.kbytes, (uint32_t)(16 * p.kbytes))
                   : make_rsrc(p.B + (int64_t)n0 * p.ldb, (uint32_t)((rows_b - 1) * p.ldb + kbytes_b));
    unsigned a_row[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int r = 16 * i + r16;
        a_row[i] = r < rows_a ? (unsigned)(r * p.lda) : OOB;
    }
    const unsigned b_row = r16 < rows_b ? (unsigned)(r16 * p.ldb) : OOB;
    const unsigned b_slot = 16u * (4 * r16 + (g ^ ((r16 >> 2) & 3)));   // packed: this lane's slot

    const int ksteps = (p.kbytes + T::KSTEP - 1) / T::KSTEP;
    const int nst = ksteps > wave ? (ksteps - wave + SK_WAVES - 1) / SK_WAVES : 0;

    // MX scale rows: A row 16i + l%16; B row l%16 (1x32) or its 32-row group.
    // Blockscale: fp32 rows of K/128 values (K/32 bytes): A row 16i + l%16,
    // B row n0/128 (the same for the whole workgroup).
    __amdgpu_buffer_rsrc_t rsa, rsb;
    unsigned sa_row[TM], sb_row = OOB;
    if constexpr (INK) {
        rsa = make_rsrc(p.mx_sa + (int64_t)m0 * p.kblocks, (uint32_t)(rows_a * p.kblocks));
        const int sb0 = n0 / BROWS, sb_rows = (n0 + rows_b - 1) / BROWS - sb0 + 1;
        rsb = make_rsrc(p.mx_sb + (int64_t)sb0 * p.kblocks, (uint32_t)(sb_rows * p.kblocks));
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r = 16 * i + r16;
            sa_row[i] = r < rows_a ? (unsigned)(r * p.kblocks) : OOB;
        }
        if (r16 < rows_b)
            sb_row = (unsigned)(((n0 + r16) / BROWS - sb0) * p.kblocks);
    }

    Frag fa[D][TM], fb[D];
    unsigned ssa[INK ? D : 1][TM], ssb[INK ? D : 1];
    Acc acc[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i)
        acc[i] = Acc{};

    // Fragments of this wave's step j into ring slot SLOT (zeros past K).
    auto load = [&](auto slotc, int j) {
        constexpr int SLOT = decltype(slotc)::value;
        const int s = wave + SK_WAVES * j;
#pragma unroll
        for (int c = 0; c < T::NCH; ++c) {
            const int kc = s * T::KSTEP + 64 * c + 16 * g;
            const bool kin = s < ksteps && kc < p.kbytes;
            if constexpr (B4) {
                // one 16-byte e2m1 chunk per lane and step; VGPRs 4-7 unused
                if (c == 0) {
                    const int kcb = s * 64 + 16 * g;
                    const u32x4 vb = ld16(rb, (s < ksteps && kcb < kbytes_b) ? b_row + (unsigned)kcb : OOB);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        fb[SLOT][q] = (int)vb[q];
                        fb[SLOT][4 + q] = 0;
                    }
                }
            } else {
                const unsigned bo = p.b_packed ? b_slot + (unsigned)((s * T::KSTEP + 64 * c) / 64) * 1024u
                                               : b_row + (unsigned)kc;
                const u32x4 vb = ld16(rb, kin ? bo : OOB);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    fb[SLOT][4 * c + q] = (int)vb[q];
            }
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const u32x4 va = ld16(ra, kin ? a_row[i] + (unsigned)kc : OOB);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    fa[SLOT][i][4 * c + q] = (int)va[q];
            }
        }
        if constexpr (MX) {
            // block g of step s; past K/32 (or past the wave's steps) reads 0
            const int kblk = 4 * s + g;
            const bool bin = s < ksteps && kblk < p.kblocks;
            ssb[SLOT] = __builtin_amdgcn_raw_buffer_load_b8(rsb, bin ? sb_row + (unsigned)kblk : OOB, 0, 0);
#pragma unroll
            for (int i = 0; i < TM; ++i)
                ssa[SLOT][i] = __builtin_amdgcn_raw_buffer_load_b8(rsa, bin ? sa_row[i] + (unsigned)kblk : OOB, 0, 0);
        } else if constexpr (BS) {
            // block s: fp32 word s of each scale row (0 past K/128)
            const bool bin = s < ksteps;
            ssb[SLOT] = __builtin_amdgcn_raw_buffer_load_b32(rsb, bin ? (unsigned)(4 * s) : OOB, 0, 0);
#pragma unroll
            for (int i = 0; i < TM; ++i)
                ssa[SLOT][i] = __builtin_amdgcn_raw_buffer_load_b32(rsa, bin ? sa_row[i] + (unsigned)(4 * s) : OOB,
                                                                    0, 0);
        }
    };
    auto mma = [&](auto slotc) {
        constexpr int SLOT = decltype(slotc)::value;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if constexpr (PATH == PATH_I8) {
                acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fb[SLOT], fa[SLOT][i], acc[i], 0, 0, 0);
            } else if constexpr (PATH == PATH_F8) {
                acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[SLOT], fa[SLOT][i], acc[i], 0, 0,
                                                                          0, 0, 0, 0);
            } else if constexpr (PATH == PATH_MX8) {
                acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    fb[SLOT], fa[SLOT][i], acc[i], 0, 0, 0, (int)ssb[SLOT], 0, (int)ssa[SLOT][i]);
            } else if constexpr (PATH == PATH_MX84) {
                acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    fb[SLOT], fa[SLOT][i], acc[i], 4, 0, 0, (int)ssb[SLOT], 0, (int)ssa[SLOT][i]);
            } else if constexpr (PATH == PATH_F8B) {
                const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[SLOT], fa[SLOT][i], f32x4{},
                                                                                   0, 0, 0, 0, 0, 0);
                const float w = __builtin_bit_cast(float, ssa[SLOT][i]) * __builtin_bit_cast(float, ssb[SLOT]);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[i][r] = __builtin_fmaf(part[r], w, acc[i][r]);
            } else {
                const i32x4 b4 = fb[SLOT], a4 = fa[SLOT][i];
                const i32x8 b8 = {b4[0], b4[1], b4[2], b4[3], 0, 0, 0, 0};
                const i32x8 a8 = {a4[0], a4[1], a4[2], a4[3], 0, 0, 0, 0};
                acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b8, a8, acc[i], 4, 4, 0, (int)ssb[SLOT],
                                                                          0, (int)ssa[SLOT][i]);
            }
        }
    };

    static_for<0, D>([&](auto sc) { load(sc, decltype(sc)::value); });
    // Steps past the wave's last load zeros and add exact zeros.
    for (int j0 = 0; j0 < nst; j0 += D) {
        static_for<0, D>([&](auto sc) {
            mma(sc);
            load(sc, j0 + decltype(sc)::value + D);
        });
    }

    // Partial sums of waves 1..7 through LDS; wave 0 adds them in wave order.
    __shared__ __attribute__((aligned(16))) int red[SK_WAVES - 1][TM][4][64];
    if (wave > 0) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                // (a scalar copy first: clang's bit_cast of an ext_vector
                // element reads element 0)
                const auto e = acc[i][r];
                red[wave - 1][i][r][lane] = __builtin_bit_cast(int, e);
            }
    }
    __syncthreads();
    if (wave != 0)
        return;
#pragma unroll
    for (int w = 0; w < SK_WAVES - 1; ++w)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int v = red[w][i][r][lane];
                if constexpr (PATH == PATH_I8)
                    acc[i][r] += v;
                else
                    acc[i][r] += __builtin_bit_cast(float, v);
            }

    // Epilogue (the fixed-order binary32 sequence of the main kernels).
    const int nloc = 4 * g;
    __amdgpu_buffer_rsrc_t rsbe, rsae, rbias;
    if constexpr (!INK) {
        rsbe = make_rsrc(p.scale_b + n0, (uint32_t)(rows_b * 4));
        rsae = make_rsrc(p.scale_a + m0, (uint32_t)(rows_a * 4));
    }
    if constexpr (BIAS)
        rbias = make_rsrc(p.bias + n0, (uint32_t)(rows_b * 2));
    unsigned sbw[4] = {0, 0, 0, 0}, bbw[4] = {0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const bool in = nloc + r < rows_b;
        if constexpr (!INK)
            sbw[r] = __builtin_amdgcn_raw_buffer_load_b32(rsbe, in ? (unsigned)((nloc + r) * 4) : OOB, 0, 0);
        if constexpr (BIAS)
            bbw[r] = (unsigned)__builtin_amdgcn_raw_buffer_load_b16(rbias, in ? (unsigned)((nloc + r) * 2) : OOB, 0,
                                                                  0) << 16;
    }
    const __amdgpu_buffer_rsrc_t rc = make_rsrc((const uint8_t *)p.C + (int64_t)m0 * p.ldc * 2,
                                                (uint32_t)((int64_t)rows_a * p.ldc * 2));
    const bool full_n = nloc + 4 <= rows_b;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int mloc = 16 * i + r16;
        float sa = 1.0f;
        if constexpr (!INK)
            sa = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                               rsae, mloc < rows_a ? (unsigned)(mloc * 4) : OOB, 0, 0));
        float f[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float x;
            if constexpr (PATH == PATH_I8)
                x = (float)acc[i][r];
            else
                x = acc[i][r];
            if constexpr (!INK) {
                x = x * sa;
                x = x * __builtin_bit_cast(float, sbw[r]);
            }
            if constexpr (BIAS)
                x = x + __builtin_bit_cast(float, bbw[r]);
            f[r] = x;
        }
        const u32x2 v = {pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3])};
        const unsigned off = mloc < rows_a ? (unsigned)((int64_t)mloc * p.ldc * 2 + (n0 + nloc) * 2) : OOB;
        if (full_n) {
            __builtin_amdgcn_raw_buffer_store_b64(v, rc, off, 0, 0);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(v[r >> 1] >> (16 * (r & 1))), rc,
                                                      (nloc + r < rows_b) ? off + 2 * r : OOB, 0, 0);
        }
    }
}

}  // namespace qgemm
