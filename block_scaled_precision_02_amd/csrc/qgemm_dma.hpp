// qgemm_dma.hpp -- the scaled GEMM with operands fetched straight into LDS.
//
// Same computation, tile geometry, fragment maps and epilogue as
// qgemm_kernel.hpp, with a different way of filling LDS:
//
//  * K advances 64 bytes per stage and LDS holds DNST = 4 stages.  Each
//    stage of A and B is fetched with buffer_load_dwordx4 ... lds (the data
//    goes from memory to LDS without passing through VGPRs), three stages
//    ahead of its use: the wave issues no LDS writes and holds no staging
//    registers, and the fetch of stage t+3 overlaps the MFMAs of stages
//    t..t+2.
//  * The kernel waits for a stage with s_waitcnt vmcnt(n), n counting the
//    loads the wave issued after the stage it needs, then a barrier (every
//    wave waited for its own share).  Fetches are spread between the MFMAs
//    (a burst of them stalls the wave's instruction issue, and with it the
//    matrix core, while the address unit works through them).
//  * MX scales arrive the same way: 16 bytes of each scale row (the scales of
//    four stages) per fetch, double-buffered, fetched four stages ahead; the
//    scale words are read from LDS together with the fragments.
//  * Blockscale FP8 (fp32 scales per 128-element K block: A [M, K/128], B
//    [ceil(N/128), K/128]) has scale rows of K/32 bytes, as long as an e4m3
//    MX scale row, and a round of four stages covers two of its blocks in 8
//    bytes of each row, as it covers eight MX blocks: its scales are staged
//    exactly like the e4m3 MX scales.  A block is two stages; its MFMAs
//    accumulate into a partial sum that starts at zero, and after the
//    block's second stage each lane folds it into the total with
//    fma(partial, sa[m, kb] * sb[n/128, kb], total) (a lane's 32x32 result
//    tile has one row m and lies inside one 128-column block).
//  * Mixed MX, e4m3 A with e2m1 B: a stage is still 64 K elements, which are
//    64 bytes of an A row and 32 bytes of a B row.  B stages hold rows of 32
//    bytes (chunk c of row r at slot c ^ ((r >> 3) & 1): 16 lanes on 16 rows
//    at one chunk cover 16 slots of 256 bytes of banks); a B fetch covers 32
//    rows.  Lane half h's 16 bytes of a B row are the instruction's K block h
//    (32 e2m1 elements, scale of lane half h), as its e4m3 A fragment's chunks
//    h and 2+h are; both operands' scales are staged as for e4m3 MX.
//  * 6-bit MX (FP6): a stage is 64 K elements, 48 bytes of a row, which is not
//    a whole 64-byte memory segment.  The ring holds segments instead
//    ("lines": 64 bytes of every row, laid out and fetched exactly as an
//    8-bit stage), four in LDS; a round of four stages spans three lines,
//    and each stage reads its fragments out of the one or two lines that
//    hold its 48 bytes.  Every segment is fetched once, whole.
//  * A 16-byte chunk c of staged row r sits at slot c ^ ((r >> 2) & 3) of its
//    64-byte row, so a fragment read (16 lanes on 16 consecutive rows at one
//    logical chunk) covers 16 different 16-byte slots of 256 bytes of banks.
//    A fetch instruction writes 1 KB of LDS (16 rows); lane i lands at
//    byte 16i of it, so lane i fetches the chunk that belongs in slot i%4 of
//    row i/4.
//
// Requirements (checked on the host, which otherwise uses qgemm_kernel):
// K bytes a whole number of stages (64 bytes), and for the scaled paths scale
// rows of whole dwords (K % 128) -- except in the SU form of the e4m3-staged
// MX paths, which takes any K % 32 (a last half stage, scale rows off dword
// boundaries).  A last round of fewer than four stages fetches the rest
// through descriptors of empty range (zeros) and replaces their scale words
// by neutral ones.  Rows past M / N are fetched from out of
// range offsets; whatever lands in LDS for them only reaches output rows and
// columns that are never stored.
#pragma once
#include "qgemm_kernel.hpp"

namespace qgemm {

constexpr int DSTAGE = 64;   // K bytes per stage
constexpr int DNST = 4;      // stages resident in LDS

__device__ __forceinline__ int dlds_off(int r, int c)
{
    return r * DSTAGE + ((c ^ ((r >> 2) & 3)) << 4);
}

typedef __attribute__((address_space(3))) void *lds_ptr;

// One wave-wide 16-byte-per-lane fetch into LDS at dst + 16 * lane (dst is
// wave-uniform; it becomes M0).  The compiler sees a vector memory load, so
// it can interleave fetches with the MFMAs; it inserts no wait for the LDS
// data, which the kernel waits for itself (s_waitcnt vmcnt + barrier).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, unsigned voff, uint8_t *dst)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)dst, 16, voff, 0, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

template <int PATH> struct DmaTraits;
// sub-steps per 64-byte stage and the chunk (of 4) a lane half reads
template <> struct DmaTraits<PATH_I8> { static constexpr int NSUB = 2; };   // chunk 2S+h
template <> struct DmaTraits<PATH_F8> { static constexpr int NSUB = 1; };   // chunks h, 2+h
template <> struct DmaTraits<PATH_MX8> { static constexpr int NSUB = 1; };  // chunks h, 2+h
template <> struct DmaTraits<PATH_MX4> { static constexpr int NSUB = 2; };  // chunk 2h+S
template <> struct DmaTraits<PATH_F8B> { static constexpr int NSUB = 1; };  // chunks h, 2+h
template <> struct DmaTraits<PATH_MX84> { static constexpr int NSUB = 1; }; // A chunks h, 2+h; B chunk h of 32 B
template <> struct DmaTraits<PATH_MX48> { static constexpr int NSUB = 1; }; // A chunk h of 32 B; B chunks h, 2+h
template <> struct DmaTraits<PATH_MX4H> { static constexpr int NSUB = 1; }; // A and B chunk h of 32 B
template <> struct DmaTraits<PATH_MX6> { static constexpr int NSUB = 1; };  // 24 bytes at 24h of a 48-byte row
template <> struct DmaTraits<PATH_MX6E3> { static constexpr int NSUB = 1; };

// Fragment of a 32-byte staged e2m1 row (the mixed paths' e2m1 operand):
// lane half h's 16 bytes (32 elements); VGPRs 4-7 unused.  HALF < 0: the
// one-stage layout (chunk c of row r at slot c ^ ((r >> 3) & 1) of 32 bytes);
// else stage HALF of a pair: 64-byte rows holding the pair's two stages,
// logical chunk q = 2 * HALF + c at slot q ^ ((r >> 2) & 3), so that 16 lanes
// on 16 consecutive rows at one chunk cover 16 different 16-byte slots of
// 256 bytes of banks.
template <int HALF = -1>
__device__ __forceinline__ i32x8 dma_frag_b32(const uint8_t *tile, int row, int h)
{
    const int off = HALF < 0 ? row * 32 + ((h ^ ((row >> 3) & 1)) << 4)
                             : row * 64 + (((2 * HALF + h) ^ ((row >> 2) & 3)) << 4);
    const i32x4 lo = *(const i32x4 *)(tile + off);
    return i32x8{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
}

// Fragment of a 32-row MFMA operand for sub-step S of a 64-byte stage.
//   int8:  16 bytes, chunk 2S+h (32 elements per sub-step)
//   e4m3:  32 bytes; VGPRs 0-3 form the instruction's first 32-element block
//          with the other lane half, VGPRs 4-7 the second: chunk h -> block 0,
//          chunk 2+h -> block 1 of the stage; lane half h's scale is block h's.
//   e2m1:  16 bytes = one 32-element block, chunk 2h+S (block 2h+S); lane
//          half h's scales are blocks 2h and 2h+1 of the stage.
// Pair layout: two consecutive stages share a 128-byte row segment, logical
// chunk q = 4 * (stage % 2) + c of row r at slot q ^ ((r >> 1) & 7), so that
// 16 lanes on 16 consecutive rows at one logical chunk cover 16 different
// 16-byte slots of 256 bytes of banks.
__device__ __forceinline__ int plds_off(int r, int q)
{
    return r * 128 + ((q ^ ((r >> 1) & 7)) << 4);
}

// HALF < 0: the one-stage layout (dlds_off); else the stage's half of the
// pair layout.
template <int PATH, int S, int HALF>
__device__ __forceinline__ typename PathTraits<PATH>::Frag dma_frag(const uint8_t *tile, int row, int h)
{
    auto off = [&](int c) { return HALF < 0 ? dlds_off(row, c) : plds_off(row, 4 * HALF + c); };
    typename PathTraits<PATH>::Frag f;
    if constexpr (PATH == PATH_I8) {
        f = *(const i32x4 *)(tile + off(2 * S + h));
    } else if constexpr (PATH == PATH_MX4) {
        i32x4 lo = *(const i32x4 *)(tile + off(2 * h + S));
        f = i32x8{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
    } else {
        i32x4 lo = *(const i32x4 *)(tile + off(h));
        i32x4 hi = *(const i32x4 *)(tile + off(2 + h));
        f = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    return f;
}

// WN = 2: 4 waves (one per SIMD) of 128x128; WN = 4: 8 waves (two per
// SIMD, so one can issue MFMAs while the other waits) of 128x64.
// SU (the e4m3-staged MX paths at K % 128 != 0): scale rows of K/32 bytes
// that start off dword boundaries, and at K % 64 == 32 a last stage of 32 K
// elements.  (One kernel template: the body moved into a device function
// called from two kernels spilled.)
template <int PATH, int WN, int TM, int TN, bool BIAS, int BROWS, int OUT, bool SU = false>
__global__ void __launch_bounds__(128 * WN, 1) qgemm_dma_kernel(const Params p)
{
    constexpr int WM = 2;
    constexpr int NW = WM * WN;                           // waves
    constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
    constexpr int NSUB = DmaTraits<PATH>::NSUB;
    constexpr bool F6 = (PATH == PATH_MX6 || PATH == PATH_MX6E3);   // 6-bit operands: 48-byte stages in 64-byte lines
    constexpr bool MX = (PATH == PATH_MX8 || PATH == PATH_MX4 || PATH == PATH_MX84 || PATH == PATH_MX48 ||
                         PATH == PATH_MX4H || F6);
    // 32-byte stage rows (64 e2m1 elements): B under e4m3 A, A under e4m3 B,
    // both for e2m1 in 64-element stages
    constexpr bool B4 = (PATH == PATH_MX84 || PATH == PATH_MX4H);
    constexpr bool A4 = (PATH == PATH_MX48 || PATH == PATH_MX4H);
    constexpr bool BS = (PATH == PATH_F8B);               // blockscale FP8
    constexpr bool SCL = MX || BS;                        // scale chunks staged through LDS
    static_assert(!BS || BROWS == 128, "blockscale B scales cover 128 rows");
    static_assert(BROWS == 1 || (BN % BROWS == 0 || BROWS == 32), "B scale rows must align with the tile");
    // bytes per row of one ring slot (FP6: a line, 64 bytes as for 8 bits)
    constexpr int ASTAGE = A4 ? DSTAGE / 2 : DSTAGE;
    constexpr int BSTAGE = B4 ? DSTAGE / 2 : DSTAGE;
    constexpr int AROWS_PER_FETCH = 1024 / ASTAGE;       // rows one 1 KB A fetch covers
    constexpr int BROWS_PER_FETCH = 1024 / BSTAGE;       // rows one 1 KB B fetch covers
    constexpr int STAGE_BYTES = BM * ASTAGE + BN * BSTAGE;
    // The 192x192 tile of the unscaled paths keeps six stages (three pairs,
    // 144 KB): pair fetches with the prefetch four stages deep (see PAIR).
    constexpr bool P6 = (PATH == PATH_I8 || PATH == PATH_F8) && WN == 2 && TM == 3 && TN == 3;
    constexpr int NSLOT = P6 ? 6 : DNST;                   // stages resident in LDS
    constexpr int OPND_BYTES = NSLOT * STAGE_BYTES;
    // MX scale chunks: per buffer, 256 rows of A and 256 rows of B (1x32) or
    // 64 (32x32 layout: BN/32 valid rows), 16 bytes each -- what four fetches
    // of 64 rows cover; rows past the tile read zeros and are never used.
    constexpr int SA_ROWS = 256;
    constexpr int SB_ROWS = (BROWS == 1) ? 256 : 64;
    constexpr int SCL_BUF = (SA_ROWS + SB_ROWS) * 16;
    // Wide scale staging (MX with 1x32 B scales, where the wave count and LDS
    // allow): a refill brings two rounds of every scale row -- 32 bytes for
    // e2m1 (16 a round), 16 for the formats with 8 a round -- so that no
    // fetched scale byte goes unused (the narrow chunk below is 16 bytes a
    // round whatever the format).  e2m1 takes two lanes per row, 32 rows per
    // fetch; the others one lane per row, 64 rows per fetch.  Refill v
    // (rounds 2v, 2v+1) goes out in two halves, at the first stage of rounds
    // 2v-2 and 2v-1, into the buffer refill v-2 used: every round still
    // issues the same number of scale fetches per wave, so the wait counts
    // are those of the narrow scheme.  Buffer rows: the tile's A rows, then
    // its B rows.
    constexpr int RB = (PATH == PATH_MX4) ? 16 : 8;       // scale bytes per row and round
    constexpr int G = 2;                                  // rounds per wide refill
    constexpr int RW = RB * G;                            // bytes per row and refill
    constexpr int LPR = RW / 16, WRPF = 64 / LPR;         // lanes per row, rows per fetch
    constexpr int SAW = BM, SBW = BN;
    constexpr int WIDE_BUF = (SAW + SBW) * RW;
    constexpr bool PRM = OUT == OUT_BF16 && (!SCL || BIAS);
    constexpr int NWA = SAW / WRPF, NWT = NWA + SBW / WRPF;   // fetches per refill: A rows, all
    constexpr bool WIDE = !SU && MX && BROWS == 1 && SAW % WRPF == 0 && SBW % WRPF == 0 && NWT % (G * NW) == 0 &&
                          NSLOT * STAGE_BYTES + 2 * WIDE_BUF + (PRM ? PRM_BYTES : 0) <= 160 * 1024;
    constexpr int NSCW = NWT / (G * NW);                  // per wave and round
    // Unaligned scale rows (SU): every chunk is fetched from its row's
    // start rounded down to a dword, m = 1..3 bytes early on the rows that
    // start inside one; the narrow chunk's 16 bytes still hold the round's 8
    // from byte m, which the reader shifts out.
    static_assert(!SU || (MX && !F6 && RB == 8 && !WIDE), "unaligned scale rows: e4m3-staged MX, narrow chunks");
    constexpr int SCL_BYTES = SCL ? 2 * (WIDE ? WIDE_BUF : SCL_BUF) : 0;
    constexpr int NQ = TM * TN;
    constexpr int RPF = (PATH == PATH_F8 || PATH == PATH_MX8 || PATH == PATH_F8B || PATH == PATH_MX84 ||
                         PATH == PATH_MX48 || PATH == PATH_MX4H) ? 2 : 1;
    constexpr int RPF_A = A4 ? 1 : RPF, RPF_B = B4 ? 1 : RPF;
    constexpr int NDSR = TM * RPF_A + TN * RPF_B;         // fragment reads per sub-step
    constexpr int DMA_A = BM / AROWS_PER_FETCH / NW, DMA_B = BN / BROWS_PER_FETCH / NW; // fetches per wave per stage
    constexpr int NDMA = DMA_A + DMA_B;                   // fetches per wave per stage (FP6: per line)
    // Pair fetches (the eight-wave 256x256 tile of INT8, and of e2m1 with
    // 1x32 B scales -- with 32x32 ones it would spill): one
    // instruction brings 8 rows x 128 bytes -- two stages of each row, whole
    // 128-byte lines -- into the pair layout (plds_off), so a row-major
    // operand goes out as 128-byte requests instead of 64-byte halves (the
    // L2 request count halves; prepacked B, already fetched as whole lines,
    // is gathered from its blocks into the same layout).  Pair k = stages 2k,
    // 2k+1 in double slot k % 2; a pair can only be issued once both of its
    // slots are free, i.e. after the barrier of the odd stage before, so the
    // fetch runs two stages ahead instead of three: the eight-wave tile's
    // longer stages hide that, the four-wave tiles' do not (one MI355X,
    // alternating: INT8 30000x21504x5376 3.162 -> 2.999 ms moving from tile
    // 4 to tile 5 with pairs, MXFP4 8192^3 0.291 -> 0.276 ms; FP8
    // 4096x2112x7168 on the four-wave 192x192 tile 0.075 -> 0.082, INT8
    // 256x256x512 on 128x128 5.4 -> 6.1 us).
    // With six slots (P6) the pairs sit in three double slots, pair k in
    // k % 3, and pair m+3 goes out at stage 2m+1, four stages before use.
    // The mixed and 64-element-stage e2m1 paths pair their 256x256 tiles as
    // well: e4m3 rows as above, 32-byte e2m1 rows as 16 rows x 64 bytes per
    // instruction (two stages of a row: one whole 64-byte segment instead of
    // half of one).  One MI355X, alternating: e4m3 x e2m1 8192^3 0.4227 ->
    // 0.4100 ms, e2m1 x e4m3 0.4416 -> 0.4130, e2m1 8192x8192x8256 (tile 5)
    // 0.5079 -> 0.4283; with a prepacked B, already whole lines, the shorter
    // prefetch costs 0.3903 -> 0.4026 ms.  (The eight-wave e4m3 x e2m1 tile
    // with 32x32 B scales would spill: one-stage fetches there.)
    constexpr bool PAIR4 = (PATH == PATH_MX84 || PATH == PATH_MX48 || PATH == PATH_MX4H) && TM == 4 &&
                           ((WN == 4 && TN == 2 && !(PATH == PATH_MX84 && BROWS == 32)) || (WN == 2 && TN == 4));
    constexpr bool PAIR = ((PATH == PATH_I8 || (PATH == PATH_MX4 && BROWS == 1)) && WN == 4 && TM == 4 && TN == 2) ||
                          P6 || PAIR4;
    constexpr int PRA = A4 ? 16 : 8, PRB = B4 ? 16 : 8;    // rows per pair fetch instruction: A, B
    constexpr int DPA = BM / PRA / NW, DPB = BN / PRB / NW;   // pair fetches per wave: A, B
    constexpr int NPF = PAIR ? DPA + DPB : 0;
    // INT8 four-slot pair ring: a pair's fetches go out in two halves, the
    // first in region B of the odd stage whose barrier freed its slot, the
    // second in region A of the even stage after it, so that the data unit
    // takes them over two regions instead of one burst (its queue, full,
    // stalls every wave that issues a load); the pair is waited for one stage
    // later.  (One MI355X, alternating: INT8 30000x21504x5376 2.890 -> 2.852
    // ms, and 3.052 -> 2.998 ms on a slower machine; e2m1 8192^3 0.2675 -> 0.2690
    // ms, and unchanged with only the pair issued at J = 1 split, so it keeps
    // whole pairs.)
    constexpr bool PH = PAIR && !P6 && PATH == PATH_I8;
    static_assert(!PH || NPF % 2 == 0, "pair fetches split in two halves");
    static_assert(!PAIR || (DPA * PRA * NW == BM && DPB * PRB * NW == BN), "pair fetches: whole row groups");
    static_assert(!P6 || !SCL, "six-slot ring: unscaled paths only (the scale rounds are four stages)");
    // scale fetches per wave per chunk: 4 waves fetch A and B scale rows,
    // 8 waves split them (waves 0-3 A, 4-7 B)
    constexpr int NSCD = SCL ? (WIDE ? NSCW : 8 / NW) : 0;
    // A rows of a stage are fetched one region earlier than its B rows
    // (region B of the stage 4 back) except for MX, whose region B is busy
    // with scale reads.
    constexpr bool SPLIT = !SCL;
    static_assert((DMA_A * AROWS_PER_FETCH * NW == BM && DMA_B * BROWS_PER_FETCH * NW == BN),
                  "tile rows must be a whole number of fetches per wave");
    static_assert(BM <= SA_ROWS && (BROWS == 1 ? BN <= SB_ROWS : BN / 32 <= SB_ROWS), "scale rows per buffer");
    using Frag = typename PathTraits<PATH>::Frag;
    using Acc = typename AccT<PATH>::T;

    // the epilogue's output stash (whole-row stores) reuses the operand and
    // scale buffers; the mixed path's smaller B stages leave less than the
    // 256x256 stash needs, so its block is sized up to that
    constexpr int STASH_NEED = NW * TM * 32 * pow2_at_least(TN * 32 * 2 / 16) * 16;
    constexpr int BODY = (B4 || A4 || F6) ? (OPND_BYTES + SCL_BYTES > STASH_NEED ? OPND_BYTES + SCL_BYTES : STASH_NEED)
                                    : OPND_BYTES + SCL_BYTES;
    constexpr int PRM_OFF = BODY;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[BODY + (PRM ? PRM_BYTES : 0)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int h = lane >> 5, r32 = lane & 31;

    int tm, tn;
    tile_of(p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int rows_a = min(BM, p.M - m0), rows_b = min(BN, p.N - n0);

    // K is a whole number of stages (SU: possibly ending in half a stage);
    // the last round may hold fewer than four.  Its stages at or past K are
    // fetched through descriptors of empty range (zeros land in LDS, whatever
    // the offset), so their MFMAs add nothing.  FP6: nst counts the 48-byte
    // stages that the MFMAs take, nfetch the 64-byte lines that hold them
    // (the last one possibly half past K).
    const int nst = F6 ? p.K / 64 : SU ? (p.kbytes + DSTAGE - 1) / DSTAGE : p.kbytes / DSTAGE;
    const int nfetch = F6 ? (p.kbytes + DSTAGE - 1) / DSTAGE : nst;
    const uint8_t *const a_base = p.A + (int64_t)m0 * p.lda;
    const int kbytes_a = A4 ? p.kbytes / 2 : p.kbytes;   // (A4 / B4: p.kbytes is K, a byte per element)
    const uint32_t a_range = (uint32_t)((rows_a - 1) * p.lda + kbytes_a);
    // B row-major, or prepacked: 16-row groups of 1 KB blocks (32-row groups
    // for the mixed path's 32-byte B rows), block t of a group holding its
    // rows' K piece t already in this kernel's LDS order, so that a fetch
    // reads one contiguous kilobyte.
    constexpr int PGR = BROWS_PER_FETCH;                  // rows per packed group
    const int kbytes_b = B4 ? p.kbytes / 2 : p.kbytes;
    const int64_t gbytes = (int64_t)PGR * kbytes_b;       // one packed group
    const uint8_t *const b_base = p.b_packed ? p.B + (int64_t)(n0 / PGR) * gbytes : p.B + (int64_t)n0 * p.ldb;
    const uint32_t b_range = p.b_packed ? (uint32_t)(((rows_b + PGR - 1) / PGR) * gbytes)
                                        : (uint32_t)((rows_b - 1) * p.ldb + kbytes_b);
    const unsigned bstep = p.b_packed ? 1024u : (unsigned)BSTAGE;   // B bytes per stage along K

    // Fetch map: wave w's j-th A fetch covers rows 16*(4w+j) .. +15; lane i
    // takes row +i/4 and the chunk that belongs in slot i%4.  A row past M / N
    // gets offset OOB; OOB plus any K offset stays beyond the range (which is
    // below 2^31), so its fetches read zeros without a per-fetch select.
    unsigned a_off[DMA_A], b_off[DMA_B];
#pragma unroll
    for (int j = 0; j < DMA_A; ++j) {
        if constexpr (A4) {
            // 32 rows of 32 bytes (as the mixed path's B): lane i takes row
            // i/2, the chunk of slot i%2
            const int r4 = AROWS_PER_FETCH * (DMA_A * wave + j) + (lane >> 1);
            const int c4 = (lane & 1) ^ ((r4 >> 3) & 1);
            a_off[j] = r4 < rows_a ? (unsigned)(r4 * p.lda + 16 * c4) : OOB;
        } else {
            const int r = 16 * (DMA_A * wave + j) + (lane >> 2);
            const int c = (lane & 3) ^ ((r >> 2) & 3);
            a_off[j] = r < rows_a ? (unsigned)(r * p.lda + 16 * c) : OOB;
        }
    }
#pragma unroll
    for (int j = 0; j < DMA_B; ++j) {
        const int g = DMA_B * wave + j;                   // 16-row group in the tile
        const int r = 16 * g + (lane >> 2);
        const int c = (lane & 3) ^ ((r >> 2) & 3);
        if constexpr (B4) {
            // 32 rows of 32 bytes: lane i takes row i/2, the chunk of slot i%2
            // (prepacked: slot i of the group's block)
            const int r4 = BROWS_PER_FETCH * g + (lane >> 1);
            const int c4 = (lane & 1) ^ ((r4 >> 3) & 1);
            if (p.b_packed)
                b_off[j] = PGR * g < rows_b ? (unsigned)(g * gbytes + 16 * lane) : OOB;
            else
                b_off[j] = r4 < rows_b ? (unsigned)(r4 * p.ldb + 16 * c4) : OOB;
        } else if (p.b_packed) {
            b_off[j] = 16 * g < rows_b ? (unsigned)(g * gbytes + 16 * lane) : OOB;
        } else {
            b_off[j] = r < rows_b ? (unsigned)(r * p.ldb + 16 * c) : OOB;
        }
    }
    // Pair fetch map: wave w's j-th A pair fetch covers rows 8*(DPA*w + j) ..
    // +7 (group g); lane i takes row r = 8g + i/8 and the logical chunk
    // q = (i & 7) ^ ((r >> 1) & 7) whose slot is i%8.  Bit 2 of q (chunks 4..7:
    // the pair's second stage) is bit 2 of i xor bit 0 of g: a pair whose
    // second stage is past K sends those lanes out of range.
    // 32-byte rows (A4 / B4): wave w's j-th pair fetch covers rows
    // 16*(D*w + j) .. +15; lane i takes row r = 16g + i/4 and the logical
    // chunk q = (i & 3) ^ ((r >> 2) & 3) (slot i%4 of the row's 64 bytes);
    // q >= 2 (the pair's second stage) exactly when bit 1 of i differs from
    // bit 5, whatever the group.
    unsigned pa_off[PAIR ? DPA : 1], pb_off[PAIR ? DPB : 1];
    const bool p_lb2 = (lane >> 2) & 1;
    const bool p_hi4 = ((lane >> 1) & 1) != ((lane >> 5) & 1);
    if constexpr (PAIR) {
#pragma unroll
        for (int j = 0; j < DPA; ++j) {
            if constexpr (A4) {
                const int r = 16 * (DPA * wave + j) + (lane >> 2);
                const int q = (lane & 3) ^ ((r >> 2) & 3);
                pa_off[j] = r < rows_a ? (unsigned)(r * p.lda + 16 * q) : OOB;
            } else {
                const int r = 8 * (DPA * wave + j) + (lane >> 3);
                const int q = (lane & 7) ^ ((r >> 1) & 7);
                pa_off[j] = r < rows_a ? (unsigned)(r * p.lda + 16 * q) : OOB;
            }
        }
#pragma unroll
        for (int j = 0; j < DPB; ++j) {
          if constexpr (B4) {
            const int r = 16 * (DPB * wave + j) + (lane >> 2);
            const int q = (lane & 3) ^ ((r >> 2) & 3);
            // prepacked (32-row groups of 1 KB blocks, block t = stage t of
            // the group's rows, slot p = row p/2, chunk (p & 1) ^ ((p >> 4) & 1)):
            // chunk q of pair 0 is chunk q % 2 of row r in block q / 2
            const int rr = r % 32, c = q & 1;
            const unsigned packed = (unsigned)((r / 32) * gbytes + (q >> 1) * 1024 +
                                               16 * (2 * rr + (c ^ ((rr >> 3) & 1))));
            const bool ok = p.b_packed ? 32 * (r / 32) < rows_b : r < rows_b;
            pb_off[j] = ok ? (p.b_packed ? packed : (unsigned)(r * p.ldb + 16 * q)) : OOB;
          } else {
            const int r = 8 * (DPB * wave + j) + (lane >> 3);
            const int q = (lane & 7) ^ ((r >> 1) & 7);
            // prepacked B (16-row groups of 1 KB blocks, block t = stage t of
            // the group's rows in the one-stage LDS order): chunk q of pair 0
            // is chunk q % 4 of row r in block q / 4.  The 8 rows of one fetch
            // are 512 contiguous bytes of each of the two blocks.
            const int c = q & 3;
            const unsigned packed = (unsigned)((r / 16) * gbytes + (q >> 2) * 1024 + (r % 16) * DSTAGE +
                                               ((c ^ ((r >> 2) & 3)) << 4));
            // (packed: every row of a group that holds a row below N, as the
            // one-stage map fetches whole groups)
            const bool ok = p.b_packed ? 16 * (r / 16) < rows_b : r < rows_b;
            pb_off[j] = ok ? (p.b_packed ? packed : (unsigned)(r * p.ldb + 16 * q)) : OOB;
          }
        }
    }
    const unsigned pbstep = p.b_packed ? 2048u : 2u * BSTAGE;   // B bytes per pair along K
    // SU with K % 64 == 32: the last stage holds 32 K elements -- the first
    // 32 bytes of a 64-byte stage row, the first 16 of a 32-byte one.  A
    // fetch whose lane's 16-byte chunk starts at or past its row's K bytes
    // goes out of range (zeros).  The chunk's column (bytes from the start of
    // the stage, or of the pair) is one per lane for every fetch of a map:
    // (i & 3) ^ ((i >> 4) & 3) chunks for one-stage 64-byte rows and pair
    // 32-byte rows, (i & 1) ^ ((i >> 4) & 1) for one-stage 32-byte rows, and
    // for pair 64-byte rows (i & 7) ^ ((i >> 4) & 3), bit 2 flipped in odd
    // groups -- the maps above with their row terms worked out.
    const int col64 = 16 * ((lane & 3) ^ ((lane >> 4) & 3));
    const int col32 = 16 * ((lane & 1) ^ ((lane >> 4) & 1));
    const int colp = 16 * ((lane & 7) ^ ((lane >> 4) & 3));
    auto kcut = [&](unsigned o, int col, int k0, int row_bytes) -> unsigned {
        if constexpr (SU)
            return col < row_bytes - k0 ? o : OOB;
        else
            return o;
    };
    // The v-th pair fetch of pair k (A fetches, then B).
    auto fetch_pair = [&](int k, auto vc) {
        constexpr int v = decltype(vc)::value;
        const bool live = 2 * k < nst, live_hi = 2 * k + 1 < nst;   // uniform
        uint8_t *ds = &lds[(P6 ? k % 3 : k & 1) * 2 * STAGE_BYTES];
        const int g = v < DPA ? DPA * wave + v : DPB * wave + (v - DPA);   // fetch group (uniform)
        const bool hi8 = p_lb2 != (bool)(g & 1);
        if constexpr (v < DPA) {
            const bool hi = A4 ? p_hi4 : hi8;
            const int k0 = 2 * ASTAGE * k;
            const unsigned o = SU ? kcut(pa_off[v] + (unsigned)k0, A4 ? col64 : colp ^ ((g & 1) << 6), k0, kbytes_a)
                                  : (!live_hi && hi) ? OOB : pa_off[v] + (unsigned)k0;
            dma16(make_rsrc(a_base, live ? a_range : 0u), o, ds + (DPA * wave + v) * 1024);
        } else {
            constexpr int j = v - DPA;
            const bool hi = B4 ? p_hi4 : hi8;
            // (SU: B row-major, a pair 2 * BSTAGE bytes of the row)
            const int k0 = (int)pbstep * k;
            const unsigned o = SU ? kcut(pb_off[j] + (unsigned)k0, B4 ? col64 : colp ^ ((g & 1) << 6), k0, kbytes_b)
                                  : (!live_hi && hi) ? OOB : pb_off[j] + (unsigned)k0;
            dma16(make_rsrc(b_base, live ? b_range : 0u), o, ds + BM * 2 * ASTAGE + (DPB * wave + j) * 1024);
        }
    };
    // Stage (FP6: line) t goes to slot t % 4, its A rows (part 0) and B rows
    // (part 1) fetched separately.
    auto fetch_part = [&](int t, auto partc) {
        const unsigned kb = (unsigned)(t * ASTAGE), kbb = (unsigned)t * bstep;
        const bool live = t < nfetch;
        uint8_t *slot = &lds[(t & 3) * STAGE_BYTES];
        if constexpr (decltype(partc)::value == 0) {
            const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_base, live ? a_range : 0u);
#pragma unroll
            for (int j = 0; j < DMA_A; ++j)
                dma16(ra, kcut(a_off[j] + kb, A4 ? col32 : col64, (int)kb, kbytes_a),
                      slot + (DMA_A * wave + j) * 1024);
        } else {
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(b_base, live ? b_range : 0u);
#pragma unroll
            for (int j = 0; j < DMA_B; ++j)
                dma16(rb, kcut(b_off[j] + kbb, B4 ? col32 : col64, (int)kbb, kbytes_b),
                      slot + BM * ASTAGE + (DMA_B * wave + j) * 1024);
        }
    };

    // One fetch instruction of stage t: the j-th of this wave's A (part 0) or
    // B (part 1) rows, the same load fetch_part issues as its j-th.
    auto fetch_one = [&](int t, auto partc, auto jc) {
        constexpr int j = decltype(jc)::value;
        const bool live = t < nfetch;
        uint8_t *slot = &lds[(t & 3) * STAGE_BYTES];
        if constexpr (decltype(partc)::value == 0) {
            const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_base, live ? a_range : 0u);
            const int k0 = t * ASTAGE;
            dma16(ra, kcut(a_off[j] + (unsigned)k0, A4 ? col32 : col64, k0, kbytes_a), slot + (DMA_A * wave + j) * 1024);
        } else {
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(b_base, live ? b_range : 0u);
            const int k0 = (int)bstep * t;
            dma16(rb, kcut(b_off[j] + (unsigned)k0, B4 ? col32 : col64, k0, kbytes_b),
                  slot + BM * ASTAGE + (DMA_B * wave + j) * 1024);
        }
    };

    // MX scale chunks: chunk u holds 16 bytes of every scale row; e2m1 starts
    // at byte 16u (stages 4u..4u+3 x 4 blocks), e4m3 at byte 8u (its first 8
    // bytes are stages 4u..4u+3 x 2 blocks; the rest comes again in chunk u+1).
    __amdgpu_buffer_rsrc_t rsa, rsb;
    unsigned sa_fo = OOB, sb_fo = OOB;
    if constexpr (SCL) {
        // Ranges in whole dwords: a dword the range ends inside reads as
        // zero, and under SU (K/32 not a multiple of 4) the tile's last
        // scale row may end inside one.  Such a range ends the array (the
        // last tile of A, or of B's scale rows), and the dword's other bytes
        // lie in the same page; they land past the row's K/32 scales, where
        // the round's masking replaces them.
        rsa = make_rsrc(p.mx_sa + (int64_t)m0 * p.kblocks, (uint32_t)((rows_a * p.kblocks + 3) & ~3));
        const int srows_b = (rows_b + BROWS - 1) / BROWS;
        rsb = make_rsrc(p.mx_sb + (int64_t)(n0 / BROWS) * p.kblocks, (uint32_t)((srows_b * p.kblocks + 3) & ~3));
        const int sw = NW == 8 ? (wave & 3) : wave;               // scale row group of this wave
        const int ra_row = 64 * sw + lane;                         // A scale row of this lane
        sa_fo = ra_row < rows_a ? (unsigned)(ra_row * p.kblocks) & ~3u : OOB;
        const int rb_row = BROWS == 1 ? 64 * sw + lane : lane;     // 32 / 128 rows: rows 0..63, fetched alike by every wave
        sb_fo = rb_row < srows_b ? (unsigned)(rb_row * p.kblocks) & ~3u : OOB;
    }
    // Wide: half e (0, 1) of a refill is global fetches g = e * NWT/2 + NSCW *
    // wave + k, k < NSCW; fetch g < NWA covers A scale rows WRPF*g .. +WRPF-1,
    // the others B rows; lane i takes row i/LPR, bytes 16 * (i % LPR) of the
    // refill's RW.
    unsigned sw_off[WIDE ? 2 * NSCW : 1];
    bool sw_a[WIDE ? 2 * NSCW : 1];
    int sw_dst[WIDE ? 2 * NSCW : 1];
    if constexpr (WIDE) {
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int k = 0; k < NSCW; ++k) {
                const int g = e * (NWT / 2) + NSCW * wave + k;
                const bool a = g < NWA;
                const int row = WRPF * (a ? g : g - NWA) + lane / LPR;
                sw_a[e * NSCW + k] = a;
                sw_off[e * NSCW + k] =
                    row < (a ? rows_a : rows_b) ? (unsigned)(row * p.kblocks + 16 * (lane % LPR)) : OOB;
                sw_dst[e * NSCW + k] = a ? 1024 * g : SAW * RW + 1024 * (g - NWA);
            }
    }
    // Fetch u of the scales (u = r + 1, issued in round r: narrow, round
    // r+1's 16-byte chunk of every row; wide, half r % 2 of refill r/2 + 1):
    // the k-th of the NSCD instructions a wave issues for it, which the
    // regions spread between the MFMAs -- narrow, the wave's A rows (k = 0)
    // and B rows (k = 1) with four waves, its A or B rows with eight; wide,
    // the k-th of the wave's fetches of that half.
    auto fetch_scale_one = [&](int u, auto kc) {
        constexpr int k = decltype(kc)::value;
        if constexpr (WIDE) {
            const int v = (u + 1) >> 1, e = (u - 1) & 1;
            uint8_t *base = &lds[OPND_BYTES + (v & 1) * WIDE_BUF];
            dma16(sw_a[e * NSCW + k] ? rsa : rsb, sw_off[e * NSCW + k] + (unsigned)(RW * v), base + sw_dst[e * NSCW + k]);
        } else if constexpr (SCL) {
            uint8_t *base = &lds[OPND_BYTES + (u & 1) * SCL_BUF];
            // four stages of scales: 16 bytes (e2m1) or 8 bytes (e4m3, blockscale) per row
            const unsigned kb = (unsigned)((PATH == PATH_MX4 ? 16 : 8) * u);
            if constexpr (NW == 4) {
                if constexpr (k == 0)
                    dma16(rsa, sa_fo + kb, base + 64 * 16 * wave);
                else
                    dma16(rsb, sb_fo + kb, base + SA_ROWS * 16 + (BROWS == 1 ? 64 * 16 * wave : 0));
            } else if (wave < 4) {
                dma16(rsa, sa_fo + kb, base + 64 * 16 * wave);
            } else {
                dma16(rsb, sb_fo + kb, base + SA_ROWS * 16 + (BROWS == 1 ? 64 * 16 * (wave - 4) : 0));
            }
        }
    };
    // The prologue's scale fetches: round 0's chunk (narrow); refill 0 whole,
    // both halves (wide).  Round r's own fetches (u = r + 1: narrow, round
    // r+1's chunk; wide, half r % 2 of refill r/2 + 1, so that round 2v-2
    // fetches half 0 of refill v and round 2v-1 half 1) go out one
    // instruction at a time between the MFMAs.
    auto fetch_scales0 = [&]() {
        if constexpr (WIDE) {
#pragma unroll
            for (int k = 0; k < 2 * NSCW; ++k)
                dma16(sw_a[k] ? rsa : rsb, sw_off[k], &lds[OPND_BYTES] + sw_dst[k]);
        } else if constexpr (SCL) {
            static_for<0, NSCD>([&](auto kc) { fetch_scale_one(0, kc); });
        }
    };

    Acc acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = Acc{};
    // blockscale: the current K block's partial sums and the fold factors
    // sa * sb of the stage being multiplied (use) and of the next (nxt)
    constexpr int BTM = BS ? TM : 1, BTN = BS ? TN : 1;
    Acc pacc[BTM][BTN];
    float fs_use[BTM][BTN], fs_nxt[BTM][BTN];

    const int arow = wm * TM * 32 + r32;
    const int brow = wn * TN * 32 + r32;
    Frag fa[2][TM], fb[2][TN];
    unsigned sa_use[TM], sb_use[TN], sa_nxt[TM], sb_nxt[TN];
    // the words of each scale row's chunk that cover the current round
    constexpr int SCW = (PATH == PATH_MX4) ? 4 : 2;
    unsigned cra[TM][SCW], crb[TN][SCW];

    // FP6 fragment of stage s = 4v + J for the 32-row block at `row` of the
    // part at `part` (A at 0, B at BM * 64).  The stage's bytes [48J, 48J+48)
    // of round v sit in lines 3v .. 3v+2 (line 3v + l in slot (3v + l) % 4);
    // lane half h's block is the 24 bytes at 48J + 24h, read as 16 bytes at
    // 48J + 32h and 8 bytes at 48J + 16 + 8h (both inside one line), and
    // joined in memory order: [16 | 8] for h = 0, [8 | 16] for h = 1, into
    // VGPRs 0-5 as the instruction reads a 6-bit operand (element k of the
    // block in bits 6k..6k+5, lowest bits first).  The 16-byte reads of 16
    // consecutive rows fall in 16 different bank groups; the 8-byte reads of
    // rows r and r+16 share banks (a 48-byte stage cannot give the two halves
    // of a 16-byte slot to one lane half, so one read in two is conflicted).
    // FP6 fragment reads.  Stage s = 4v + J covers bytes [48J, 48J + 48) of
    // round v, which sit in lines 3v .. 3v+2 (line 3v + l in slot
    // (3v + l) % 4).  Lane half h's block is the 24 bytes at 48J + 24h, read
    // as three 8-byte reads in memory order straight into VGPRs 0-5, as the
    // instruction takes a 6-bit operand (element k of the block in bits
    // 6k..6k+5, lowest bits first); each 8-byte read lies inside one line.
    // (One 16-byte and one 8-byte read would cost fewer LDS cycles, but
    // lane half 1's block starts 8 bytes into a 16-byte slot, and joining the
    // two reads in a half-dependent order takes six selects a fragment: the
    // wave ran out of VALU issue before LDS.)  The 8-byte reads of rows r
    // and r+16 share banks: a 16-byte-slot swizzle cannot give the two 8-byte
    // halves of a slot to one lane half, so each read takes two passes.
    //
    // Per lane and stage position J the three reads' offsets in a ring whose
    // line 3v sat in slot 0 -- line * STAGE_BYTES, the swizzled chunk, the
    // 8-byte half and the lane's row r32 -- are kept in 12 registers.  A read
    // adds the round's slot of line 3v and the wave's row block (uniform),
    // wraps at the ring's end (the within-slot part stays below STAGE_BYTES,
    // so the wrap only touches the slot bits), and takes the operand part and
    // the 32-row block as the instruction's immediate offset.
    static_assert(!F6 || (STAGE_BYTES & (STAGE_BYTES - 1)) == 0, "FP6 ring addressing");
    constexpr unsigned RING = 4u * STAGE_BYTES - 1;
    unsigned f6o[F6 ? 4 : 1][3];
    if constexpr (F6) {
        const int swx = ((r32 >> 2) & 3) << 4;
#pragma unroll
        for (int J = 0; J < 4; ++J)
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                const int b = 48 * J + 24 * h + 8 * q;   // byte of the round
                f6o[J][q] = (unsigned)((b >> 6) * STAGE_BYTES + ((b & 48) ^ swx) + (b & 8) + r32 * DSTAGE);
            }
    }
    auto f6_frag = [&](auto jc, int s, auto partc, unsigned wrow, auto blkc) -> i32x8 {
        constexpr int J = decltype(jc)::value;
        constexpr int IMM = decltype(partc)::value + 32 * decltype(blkc)::value * DSTAGE;
        const unsigned u = (unsigned)(((3 * (s >> 2)) & 3) * STAGE_BYTES) + wrow * DSTAGE;   // uniform
        const u32x2 a = *(const u32x2 *)&lds[((u + f6o[J][0]) & RING) + IMM];
        const u32x2 b = *(const u32x2 *)&lds[((u + f6o[J][1]) & RING) + IMM];
        const u32x2 c = *(const u32x2 *)&lds[((u + f6o[J][2]) & RING) + IMM];
        return i32x8{(int)a[0], (int)a[1], (int)b[0], (int)b[1], (int)c[0], (int)c[1], 0, 0};
    };

    // Fragment k of sub-step S of stage s (ring slot SLOT = s % 4; FP6: J =
    // s % 4) in the order the serpentine MFMA sequence consumes them: A row
    // block 0, the TN B column blocks, A row blocks 1..
    auto read_item = [&](auto kc, auto sc, auto slotc, auto setc, int s) {
        constexpr int k = decltype(kc)::value;
        constexpr int S = decltype(sc)::value;
        constexpr int SLOT = decltype(slotc)::value;
        constexpr int SET = decltype(setc)::value;
        // pair layout: slot SLOT is half SLOT % 2 of double slot SLOT / 2
        constexpr int HALF = PAIR ? (SLOT & 1) : -1;
        const uint8_t *ta = PAIR ? &lds[(SLOT >> 1) * 2 * STAGE_BYTES] : &lds[SLOT * STAGE_BYTES];
        const uint8_t *tb = ta + BM * (PAIR ? 2 * ASTAGE : ASTAGE);
        if constexpr (F6) {
            using P0 = std::integral_constant<int, 0>;
            using PB = std::integral_constant<int, BM * DSTAGE>;
            if constexpr (k == 0)
                fa[SET][0] = f6_frag(slotc, s, P0(), (unsigned)(wm * TM * 32), P0());
            else if constexpr (k <= TN)
                fb[SET][k - 1] = f6_frag(slotc, s, PB(), (unsigned)(wn * TN * 32), std::integral_constant<int, k - 1>());
            else
                fa[SET][k - TN] = f6_frag(slotc, s, P0(), (unsigned)(wm * TM * 32), std::integral_constant<int, k - TN>());
        } else if constexpr (k == 0) {
            if constexpr (A4)
                fa[SET][0] = dma_frag_b32<HALF>(ta, arow, h);
            else
                fa[SET][0] = dma_frag<PATH, S, HALF>(ta, arow, h);
        } else if constexpr (k <= TN) {
            if constexpr (B4)
                fb[SET][k - 1] = dma_frag_b32<HALF>(tb, brow + 32 * (k - 1), h);
            else
                fb[SET][k - 1] = dma_frag<PATH, S, HALF>(tb, brow + 32 * (k - 1), h);
        } else {
            if constexpr (A4)
                fa[SET][k - TN] = dma_frag_b32<HALF>(ta, arow + 32 * (k - TN), h);
            else
                fa[SET][k - TN] = dma_frag<PATH, S, HALF>(ta, arow + 32 * (k - TN), h);
        }
    };

    // Scale operands.  Once per round (4 stages) each lane reads the words of
    // its rows' 16-byte scale chunks that the round uses (one aligned 16- or
    // 8-byte LDS read per row: narrower per-stage reads of 32 rows at a
    // 16-byte stride land 4 rows to a bank); each stage then shifts out its
    // operand: byte S of it is sub-step S's scale for the lane's block --
    // e2m1: bytes 4J + 2h, 4J + 2h + 1 of the chunk; e4m3: byte 2J + h.
    auto load_chunk = [&](int t) {
        if constexpr (SCL) {
            // narrow: round r's 16 bytes at row * 16 of buffer r % 2; wide:
            // round r's RB bytes at row * RW + RB * (r % G) of buffer (r / G) % 2
            const int r = t >> 2;
            const uint8_t *sbuf = WIDE ? &lds[OPND_BYTES + ((r / G) & 1) * WIDE_BUF] + RB * (r % G)
                                       : &lds[OPND_BYTES + (r & 1) * SCL_BUF];
            constexpr int SP = WIDE ? RW : 16;                // row pitch
            constexpr int SBOFF = WIDE ? SAW * RW : SA_ROWS * 16;
            // (SU: the row's 8 bytes start at byte m of its chunk)
            auto rd = [&](const uint8_t *row_base, unsigned (&w)[SCW], unsigned m) {
                if constexpr (SU) {
                    const u32x4 v = *(const u32x4 *)row_base;
                    w[0] = __builtin_amdgcn_alignbyte(v[1], v[0], m);
                    w[1] = __builtin_amdgcn_alignbyte(v[2], v[1], m);
                } else if constexpr (SCW == 4) {
                    const u32x4 v = *(const u32x4 *)row_base;
#pragma unroll
                    for (int q = 0; q < 4; ++q) w[q] = v[q];
                } else {
                    const u32x2 v = *(const u32x2 *)row_base;
                    w[0] = v[0];
                    w[1] = v[1];
                }
            };
            // a row's offset in its dword (0 unless SU; rows 32 apart share it)
            const unsigned ma = SU ? (unsigned)(arow * p.kblocks) & 3u : 0u;
#pragma unroll
            for (int i = 0; i < TM; ++i)
                rd(sbuf + (arow + 32 * i) * SP, cra[i], ma);
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int row = BROWS == 1 ? brow + 32 * j : (wn * TN * 32 + 32 * j) / BROWS;
                rd(sbuf + SBOFF + row * SP, crb[j], SU ? (unsigned)(row * p.kblocks) & 3u : 0u);
            }
        }
    };
    auto neutral_chunk = [&](int t) {
        if constexpr (SCL) {
            // Words of stages past K (the last round's tail) hold the next
            // row's scales or zeros: make them finite and neutral -- scale
            // 2^0 under zero data for MX, a fold factor of 0 for blockscale.
            // Word 0 is always live (a round starts below K), and each word
            // covers 4 / SCW whole stages: outside SU the host admits only K
            // with a whole number of words (K % 128), so a word is either
            // wholly past K or wholly before it; SU splits words.
            constexpr unsigned NEUTRAL = BS ? 0u : 0x7F7F7F7Fu;
            static_assert(4 % SCW == 0, "a scale word covers whole stages");
            if constexpr (SU) {
                // K/32 not a multiple of 4: the round's last live word ends
                // in K/32 mod 4 live bytes (byte b of word w: K block
                // 2t + 4w + b); its other bytes are past K
#pragma unroll
                for (int w = 0; w < SCW; ++w) {
                    const int live = p.kblocks - 2 * t - 4 * w;   // uniform
                    const unsigned keep = live >= 4 ? ~0u : live <= 0 ? 0u : (1u << (8 * live)) - 1u;
                    const unsigned fill = NEUTRAL & ~keep;
#pragma unroll
                    for (int i = 0; i < TM; ++i) cra[i][w] = (cra[i][w] & keep) | fill;
#pragma unroll
                    for (int j = 0; j < TN; ++j) crb[j][w] = (crb[j][w] & keep) | fill;
                }
            } else {
#pragma unroll
                for (int w = 1; w < SCW; ++w) {
                    const bool past = t + w * (4 / SCW) >= nst;
#pragma unroll
                    for (int i = 0; i < TM; ++i) cra[i][w] = past ? NEUTRAL : cra[i][w];
#pragma unroll
                    for (int j = 0; j < TN; ++j) crb[j][w] = past ? NEUTRAL : crb[j][w];
                }
            }
        }
    };
    auto read_chunk = [&](int t) {
        load_chunk(t);
        neutral_chunk(t);
    };
    // (LOADED: the round's chunk words were loaded at the start of the
    // region; only their masking and the shifts remain)
    auto read_scales = [&](int t, auto jc, auto loadedc) {
        constexpr bool LOADED = decltype(loadedc)::value;
        if constexpr (BS) {
            // fold factors of the block stage J belongs to (word J/2 of the
            // round's 8 bytes); only the block's second stage folds
            constexpr int J = decltype(jc)::value;
            if constexpr (J == 0) {
                if constexpr (LOADED)
                    neutral_chunk(t);
                else
                    read_chunk(t);
            }
            if constexpr (J & 1) {
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        fs_nxt[i][j] = __builtin_bit_cast(float, cra[i][J >> 1]) *
                                       __builtin_bit_cast(float, crb[j][J >> 1]);
            }
        } else if constexpr (MX) {
            constexpr int J = decltype(jc)::value;
            if constexpr (J == 0) {
                if constexpr (LOADED)
                    neutral_chunk(t);
                else
                    read_chunk(t);
            }
            constexpr int W = (PATH == PATH_MX4) ? J : J >> 1;
            const unsigned sh = (PATH == PATH_MX4) ? 16u * h : 8u * (2 * (J & 1) + h);
#pragma unroll
            for (int i = 0; i < TM; ++i)
                sa_nxt[i] = cra[i][W] >> sh;
#pragma unroll
            for (int j = 0; j < TN; ++j)
                sb_nxt[j] = crb[j][W] >> sh;
        }
    };
    auto mfmas = [&](auto sc, auto setc, auto q0c, auto q1c, auto jc) {
        constexpr int S = decltype(sc)::value;
        constexpr int SET = decltype(setc)::value;
        constexpr int J = decltype(jc)::value;
        static_for<decltype(q0c)::value, decltype(q1c)::value>([&](auto qc) {
            constexpr int Q = decltype(qc)::value;
            constexpr int i = Q / TN;
            constexpr int j = (i & 1) ? (TN - 1 - Q % TN) : (Q % TN);
            if constexpr (BS) {
                if constexpr ((J & 1) == 0) {
                    // first stage of a K block: the partial sum starts at zero
                    pacc[i][j] = Acc{};
                    mfma<PATH, S>(pacc[i][j], fb[SET][j], fa[SET][i], 0u, 0u);
                } else {
                    // second stage: the partial sum is folded one MFMA later
                    // (fold), once the matrix core has produced it
                    mfma<PATH, S>(pacc[i][j], fb[SET][j], fa[SET][i], 0u, 0u);
                }
            } else {
                mfma<PATH, S>(acc[i][j], fb[SET][j], fa[SET][i], MX ? sb_use[j] : 0u, MX ? sa_use[i] : 0u);
            }
        });
    };
    // Blockscale, a K block's second stage: total += partial * (sa * sb) for
    // the MFMA tile Q of the serpentine order.
    auto fold = [&](auto qc) {
        if constexpr (BS) {
            constexpr int Q = decltype(qc)::value;
            constexpr int i = Q / TN;
            constexpr int j = (i & 1) ? (TN - 1 - Q % TN) : (Q % TN);
            const float f = fs_use[i][j];
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = __builtin_fmaf(pacc[i][j][e], f, acc[i][j][e]);
        }
    };
    constexpr bool FOLD_ODD = BS;   // stages J odd fold their partial sums
    // Scheduling fences after each MFMA group and at the end of each stage
    // (see stage()): kept for INT8, e2m1 and the 6-bit path.  The e4m3 paths
    // are left to the compiler's own interleaving within the same order of
    // reads and fetches (one MI355X, alternating against the fenced build:
    // blockscale 16384x7168x2048 0.305 vs 0.332 ms, e4m3 x e2m1 8192^3 0.483
    // vs 0.486, FP8 4096x2112x7168 and MXFP8 within noise; MXFP6 8192^3 0.525
    // vs 0.520 ms, so it keeps them).
    constexpr bool FENCE = NSUB == 2 || F6;
    auto use_next_scales = [&]() {
        if constexpr (BS) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) fs_use[i][j] = fs_nxt[i][j];
        } else if constexpr (MX) {
#pragma unroll
            for (int i = 0; i < TM; ++i) sa_use[i] = sa_nxt[i];
#pragma unroll
            for (int j = 0; j < TN; ++j) sb_use[j] = sb_nxt[j];
        }
    };

    // Prologue: the tile's epilogue operands (waves 0-2, one fetch each),
    // scale chunk 0, stages 0..2 and the A rows of stage 3 (FP6: lines 0..3);
    // wait for stage 0 (line 0).
    if constexpr (PRM) {
        if (wave == 0 && !SCL)
            dma16(make_rsrc(p.scale_a + m0, (uint32_t)(rows_a * 4)), 16 * lane, &lds[PRM_OFF]);
        if (wave == 1 && !SCL)
            dma16(make_rsrc(p.scale_b + n0, (uint32_t)(rows_b * 4)), 16 * lane, &lds[PRM_OFF + PRM_SB]);
        if (wave == 2 && BIAS)
            dma16(make_rsrc(p.bias + n0, (uint32_t)(rows_b * 2)), 16 * lane, &lds[PRM_OFF + PRM_BIAS]);
    }
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    // (issue order is what the wait counts: no reordering across stages)
    fetch_scales0();
    if constexpr (PAIR) {
        // pairs 0 and 1 (stages 0..3; P6: pairs 0..2; PH: pair 1's first half,
        // its second goes out in stage 0); wait for pair 0
        static_for<0, P6 ? 3 : 2>([&](auto kc) {
            constexpr int k = decltype(kc)::value;
            __builtin_amdgcn_sched_barrier(0);
            static_for<0, (PH && k == 1) ? NPF / 2 : NPF>([&](auto vc) { fetch_pair(k, vc); });
        });
    } else {
#pragma unroll
        for (int t = 0; t < (F6 ? 4 : 3); ++t) {
            __builtin_amdgcn_sched_barrier(0);
            fetch_part(t, I0());
            fetch_part(t, I1());
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (SPLIT)
            fetch_part(3, I0());
    }
    __builtin_amdgcn_sched_barrier(0);
    twin_sync();
    wait_vmcnt<PAIR ? (P6 ? 2 * NPF : PH ? NPF / 2 : NPF) : (F6 ? 3 : 2) * NDMA + (SPLIT ? DMA_A : 0)>();
    lds_barrier();
    // stage 0's first fragments (one sub-step per stage: those its first
    // half of MFMAs uses; its region A reads the rest)
    static_for<0, (NSUB == 1) ? 1 + TN + (NQ / 2 - 1) / TN : TM + TN>(
        [&](auto kc) { read_item(kc, I0(), I0(), I0(), 0); });
    read_scales(0, I0(), std::false_type());
    use_next_scales();

    // Stage t = 4q + J, in two regions of MFMAs.  Each MFMA is followed by its
    // share of the region's fragment reads and fetches, and a scheduling
    // fence keeps that order: the reads for the next MFMAs go out while the
    // current ones run (into the other register set), so the LDS latency
    // hides behind the matrix core instead of stalling the wave right before
    // the barrier or right before the MFMA that consumes them.
    //  Region A: fetch scale chunk q+1 (J == 0) and the B rows (SPLIT) or all
    //  rows of stage t+3 into the slot stage t-1 used (free since the last
    //  barrier); read sub-step 1's fragments (NSUB == 2); multiply sub-step 0
    //  (NSUB == 1: the first half of the stage's MFMAs).  Then wait for stage
    //  t+1 -- the loads issued after it are those of stages t+2 and t+3 --
    //  and meet at the barrier.
    //  Region B: fetch the A rows of stage t+4 (SPLIT) into stage t's slot
    //  (its last reads were before the barrier); read stage t+1's first
    //  fragments and its scale chunk; multiply the rest of stage t.
    auto stage = [&](int t, auto jc) {
        constexpr int J = decltype(jc)::value;             // t % 4 (P6: t % 6, the slot)
        constexpr int JN = P6 ? (J + 1) % 6 : (J + 1) & 3;
        constexpr int SET0 = (NSUB == 1) ? (J & 1) : 0;    // register set of sub-step 0
        constexpr int SETN = (NSUB == 1) ? ((J + 1) & 1) : 0;
        constexpr int NIT = TM + TN;                       // fragments per sub-step
        // One sub-step per stage (e4m3 operands): the first half of a stage's
        // MFMAs (serpentine order) uses A row blocks 0..IMAX and every B
        // column block, i.e. fragments [0, EARLY); those are read in the
        // previous stage's region B, the rest in the stage's own region A, so
        // that neither region carries a whole stage of fragment traffic.
        constexpr int IMAX = (NQ / 2 - 1) / TN;
        constexpr int EARLY = (NSUB == 1) ? 1 + TN + IMAX : NIT;
        // FP6 stages past K (the last round's tail) read what follows the
        // row's last byte in a half-live line: they are not multiplied.  The
        // other paths multiply zeros there.  (K % 128 == 0: the stage count
        // is even, so the first two stages of a round are always live.)
        // (P6: the loop runs in steps of six stages; those past K are skipped.
        // SU, whose odd stage count leaves a last round of one or three
        // stages, multiplies zeros: branching there spills the 8-wave tile.)
        const bool mul = F6 ? (J < 2 || t < nst) : P6 ? t < nst : true;
        // ---- region A
        {
            constexpr int NA = (NSUB == 2) ? NQ : NQ / 2;
            // (pairs without the INT8 halves: the scale refill goes out in
            // region B instead, which issues no pair fetch on an even stage;
            // one MI355X, alternating: e4m3 x e2m1 8192^3 0.4199 -> 0.4173 ms,
            // e2m1 8192^3 level)
            constexpr bool SCB = PAIR && !P6 && !PH;
            constexpr int NSC = (J == 0 && !SCB) ? NSCD : 0;
            constexpr int VA = SPLIT ? 0 : DMA_A;
            // pairs (four-slot ring): the second half of the pair whose first
            // half the odd stage before issued
            constexpr int NPH = (PH && (J & 1) == 0) ? NPF / 2 : 0;
            constexpr int V = NPH + NSC + ((F6 || PAIR) ? 0 : VA + DMA_B);   // fetches: pair half, scale chunk, A rows, B rows
            constexpr int R = (NSUB == 2) ? NIT : NIT - EARLY;
            constexpr int NR = NA > 2 ? NA - 2 : 1;        // reads go out before the last two MFMAs
            static_for<0, NA>([&](auto qc) {
                constexpr int Q = decltype(qc)::value;
                static_for<(Q < NR ? R * Q / NR : R), (Q < NR ? R * (Q + 1) / NR : R)>([&](auto kc) {
                    constexpr int k = decltype(kc)::value;
                    if constexpr (NSUB == 2)
                        read_item(kc, I1(), jc, I1(), t);
                    else
                        read_item(std::integral_constant<int, EARLY + k>(), I0(), jc,
                                  std::integral_constant<int, SET0>(), t);
                });
                if (mul)
                    mfmas(I0(), std::integral_constant<int, SET0>(), qc, std::integral_constant<int, Q + 1>(), jc);
                if constexpr (FOLD_ODD && (J & 1) && Q >= 1)
                    fold(std::integral_constant<int, Q - 1>());
                static_for<V * Q / NA, V * (Q + 1) / NA>([&](auto vc) {
                    constexpr int v = decltype(vc)::value;
                    if constexpr (v < NPH)
                        fetch_pair((t + 2) >> 1, std::integral_constant<int, NPF / 2 + v>());
                    else if constexpr (v < NPH + NSC)
                        fetch_scale_one((t >> 2) + 1, std::integral_constant<int, v - NPH>());
                    else if constexpr (v < NPH + NSC + VA)
                        fetch_one(t + 3, I0(), std::integral_constant<int, v - NPH - NSC>());
                    else
                        fetch_one(t + 3, I1(), std::integral_constant<int, v - NPH - NSC - VA>());
                });
                if constexpr (FENCE)
                    __builtin_amdgcn_sched_barrier(0);
            });
            if constexpr (FOLD_ODD && (J & 1))
                fold(std::integral_constant<int, NA - 1>());
        }
        // loads issued after stage t+1's: stages t+2 and t+3, plus the scale
        // chunk when it went out at stage t or t-1.  FP6 (round v, t = 4v + J;
        // issue order: line 3v+3 at stage 4v-1, scale chunk v+1 at 4v, lines
        // 3v+4..3v+6 at 4v+1..4v+3): stage t+1 needs line 3v+1 (J = 0: then
        // lines 3v+2, 3v+3 and the chunk went out), 3v+2 (J = 1: line 3v+3 and
        // the chunk), 3v+2 again (J = 2), or line 3v+3 and the chunk (J = 3:
        // then lines 3v+4, 3v+5).
        // Pairs (pair (t+3)/2's first half in region B of an odd stage t, its
        // second half in region A of stage t+1): only odd stages wait, for
        // pair (t+1)/2, whose second half went out before stage t-1's scale
        // chunk -- the one load that may still be in flight.  (Even stages:
        // the count below is unused.)  P6: stage t+1 is followed by two more
        // pairs at an even t, one at an odd t.
        constexpr int AFTER = P6 ? ((J & 1) ? 1 : 2) * NPF
                            : PAIR ? ((J & 1) ? 0 : NPF) + ((J == 0 || J == 1) ? NSCD : 0)
                            : F6   ? (J == 1 ? 1 : 2) * NDMA + (J == 3 ? 0 : NSCD)
                                   : 2 * NDMA + ((J == 0 || J == 1) ? NSCD : 0);
        // Pairs: region B of an even stage reads the second half of the pair
        // the previous (odd) stage waited for, and issues nothing; every
        // refill goes out in region B of an odd stage, after that stage's
        // barrier, into the slot whose last reads (region A of the same odd
        // stage) precede it.  So only odd stages wait and synchronise.
        constexpr bool SYNC = !(PAIR && (J & 1) == 0);
        twin_sync();
        if constexpr (SYNC) {
            wait_vmcnt<AFTER>();
            lds_barrier();
        }
        __builtin_amdgcn_sched_barrier(0);
        // ---- region B
        {
            constexpr int NB = (NSUB == 2) ? NQ : NQ - NQ / 2;
            constexpr int QB = (NSUB == 2) ? 0 : NQ / 2;   // first MFMA of the region
            // FP6: the line whose slot the barrier just freed (line 3v + J - 1,
            // last read by stage t) is refilled with line 3v + J + 3
            constexpr bool SCB = PAIR && !P6 && !PH;
            constexpr int V = PAIR ? ((J & 1) ? (PH ? NPF / 2 : NPF) : (SCB && J == 0) ? NSCD : 0)
                                   : F6 ? (J == 0 ? 0 : NDMA) : SPLIT ? DMA_A : 0;
            constexpr bool CHUNK = SCL && JN == 0;         // stage t+1 starts a round
            constexpr int R = EARLY;
            constexpr int NR = NB > 2 ? NB - 2 : 1;
            if constexpr (CHUNK)
                load_chunk(t + 1);
            static_for<0, NB>([&](auto qc) {
                constexpr int Q = decltype(qc)::value;
                static_for<(Q < NR ? R * Q / NR : R), (Q < NR ? R * (Q + 1) / NR : R)>([&](auto kc) {
                    read_item(kc, I0(), std::integral_constant<int, JN>(), std::integral_constant<int, SETN>(),
                              t + 1);
                });
                if constexpr (NSUB == 2)
                    mfmas(I1(), I1(), qc, std::integral_constant<int, Q + 1>(), jc);
                else if (mul)
                    mfmas(I0(), std::integral_constant<int, SET0>(), std::integral_constant<int, QB + Q>(),
                          std::integral_constant<int, QB + Q + 1>(), jc);
                if constexpr (FOLD_ODD && (J & 1) && Q >= 1)
                    fold(std::integral_constant<int, QB + Q - 1>());
                static_for<V * Q / NB, V * (Q + 1) / NB>([&](auto vc) {
                    constexpr int v = decltype(vc)::value;
                    if constexpr (P6)
                        fetch_pair((t + 5) >> 1, vc);
                    else if constexpr (PAIR && (J & 1))
                        fetch_pair((t + 3) >> 1, vc);
                    else if constexpr (PAIR)
                        fetch_scale_one((t >> 2) + 1, vc);
                    else if constexpr (!F6)
                        fetch_one(t + 4, I0(), vc);
                    else if constexpr (v < DMA_A)
                        fetch_one(3 * (t >> 2) + J + 3, I0(), vc);
                    else
                        fetch_one(3 * (t >> 2) + J + 3, I1(), std::integral_constant<int, v - DMA_A>());
                });
                if constexpr (FENCE)
                    __builtin_amdgcn_sched_barrier(0);
            });
            if constexpr (FOLD_ODD && (J & 1))
                fold(std::integral_constant<int, QB + NB - 1>());
            read_scales(t + 1, std::integral_constant<int, JN>(), std::true_type());
        }
        use_next_scales();
        if constexpr (FENCE)
            __builtin_amdgcn_sched_barrier(0);
        twin_sync();
        if constexpr (FENCE)
            __builtin_amdgcn_sched_barrier(0);
    };

    // The host guarantees a whole number of stages (kbytes % 64 == 0; for the
    // scaled paths, of the stages that one scale word covers; FP6: K % 128 ==
    // 0), except under SU, where the last stage may end half way (its other
    // half fetched as zeros) and the last live word part way past K.
    // Fetches run three stages (FP6: two to three lines) ahead, into stages
    // past K that are never multiplied or, in a partial last round,
    // multiplied as zeros (FP6: skipped).
    if constexpr (P6) {
        for (int t = 0; t < nst; t += 6)
            static_for<0, 6>([&](auto jc) { stage(t + decltype(jc)::value, jc); });
    } else {
        for (int t = 0; t < nst; t += 4) {
            stage(t, I0());
            stage(t + 1, I1());
            stage(t + 2, std::integral_constant<int, 2>());
            stage(t + 3, std::integral_constant<int, 3>());
        }
    }
    // Successor prefetch (e2m1 and 6-bit MX, blockscale FP8).  Once a round
    // of tiles is running, the tile that starts next on this XCD is the one of
    // workgroup blockIdx + NXT (the dispatcher hands workgroups to the 8 XCDs
    // round-robin and, within an XCD, in order to whichever CU frees up;
    // NXT = 8 XCDs x 32 CUs x the workgroups a CU holds).  Its prologue waits
    // for the first stage of its A and B rows and its first scale refill,
    // which at that point come from beyond L2.  So, with the K loop done,
    // every workgroup loads one dword of the first 128-byte line of each of
    // the next tile's A, B and scale rows (prepacked B: of the first two 1 KB
    // blocks of each row group) into registers: the lines come into the XCD's
    // L2 while this tile's epilogue runs.  The loads are range-checked like
    // every fetch and their values are never used.  They are the last loads
    // before the wait below, which therefore lets exactly them stay in
    // flight.  The launch arguments they need are read again through an
    // opaque copy of the kernarg segment pointer (the one explicit argument,
    // Params, sits at offset 0 of that segment, as the code-object ABI lays
    // explicit arguments out first), so that the K loop does not keep them in
    // registers.  (One MI355X each, alternating: MXFP4 8192^3 0.2617 -> 0.2594
    // ms on one machine, level on another, prepacked B 0.2617 -> 0.2588;
    // blockscale 16384x7168x2048 0.3200 -> 0.3152; MXFP6 8192^3 0.3947 ->
    // 0.3937.  INT8 30000x21504x5376 2.817 -> 2.837, e2m1 in 64-element stages
    // 8192x8192x8256 0.4261 -> 0.4267, MXFP8 and e4m3 x e2m1 level: those
    // paths do not prefetch.)
    constexpr bool SUCC = PATH == PATH_MX4 || F6 || BS;
    constexpr int NT = 64 * NW;
    constexpr int WPC = sizeof(lds) > 80 * 1024 ? 1 : 2;           // workgroups per CU (LDS)
    constexpr int NXT = 8 * 32 * WPC;
    constexpr int NPA = SUCC ? (BM + BN + NT - 1) / NT : 0;        // operand lines per lane
    constexpr int NPS = SUCC && SCL ? (BM + BN + NT - 1) / NT : 0; // scale lines per lane (MX / blockscale only:
                                                                   // other paths have no scale rows, and null pointers)
    unsigned pf[NPA + NPS + 1];
    typedef const Params __attribute__((address_space(4))) *KargP;
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!SUCC) {
        wait_vmcnt<0>();   // nothing may still be landing in LDS once it holds the output
    } else {
        KargP kp = (KargP)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(kp));
        const int tms = kp->tiles_m, tns = kp->tiles_n;
        const int nb = (int)blockIdx.x + NXT;
        if (nb < tms * tns) {
            int sm, sn;
            tile_of_index(tms, tns, kp->group_m, nb, sm, sn);
            const int m1 = sm * BM, n1 = sn * BN;
            const int ra = min(BM, kp->M - m1), rb = min(BN, kp->N - n1);
            const int64_t lda = kp->lda, ldb = kp->ldb;
            const __amdgpu_buffer_rsrc_t pa =
                make_rsrc(kp->A + (int64_t)m1 * lda, (uint32_t)((ra - 1) * lda + kbytes_a));
            const bool packed = kp->b_packed;
            const __amdgpu_buffer_rsrc_t pb =
                packed ? make_rsrc(kp->B + (int64_t)(n1 / PGR) * gbytes, (uint32_t)(((rb + PGR - 1) / PGR) * gbytes))
                       : make_rsrc(kp->B + (int64_t)n1 * ldb, (uint32_t)((rb - 1) * ldb + kbytes_b));
#pragma unroll
            for (int q = 0; q < NPA; ++q) {
                const int idx0 = q * NT + 64 * wave;                 // uniform: BM is a multiple of 64
                const int idx = idx0 + lane;
                if (idx0 < BM) {
                    pf[q] = __builtin_amdgcn_raw_buffer_load_b32(pa, idx < ra ? (unsigned)(idx * lda) : OOB, 0, 0);
                } else {
                    const int b = idx - BM;
                    unsigned off;
                    if (packed) {
                        // 16 lines of each group's first 2 KB
                        const int g = b >> 4;
                        off = (g < (BN + PGR - 1) / PGR && PGR * g < rb) ? (unsigned)(g * gbytes + 128 * (b & 15))
                                                                         : OOB;
                    } else {
                        off = (b < BN && b < rb) ? (unsigned)(b * ldb) : OOB;
                    }
                    pf[q] = __builtin_amdgcn_raw_buffer_load_b32(pb, off, 0, 0);
                }
            }
            if constexpr (NPS > 0) {
                const int kbl = kp->kblocks;
                const int srb = (rb + BROWS - 1) / BROWS;
                const __amdgpu_buffer_rsrc_t qa =
                    make_rsrc(kp->mx_sa + (int64_t)m1 * kbl, (uint32_t)((ra * kbl + 3) & ~3));
                const __amdgpu_buffer_rsrc_t qb =
                    make_rsrc(kp->mx_sb + (int64_t)(n1 / BROWS) * kbl, (uint32_t)((srb * kbl + 3) & ~3));
#pragma unroll
                for (int q = 0; q < NPS; ++q) {
                    const int idx0 = q * NT + 64 * wave;
                    const int idx = idx0 + lane;
                    if (idx0 < BM)
                        pf[NPA + q] = __builtin_amdgcn_raw_buffer_load_b32(
                            qa, idx < ra ? (unsigned)(idx * kbl) & ~3u : OOB, 0, 0);
                    else
                        pf[NPA + q] = __builtin_amdgcn_raw_buffer_load_b32(
                            qb, idx - BM < srb ? (unsigned)((idx - BM) * kbl) & ~3u : OOB, 0, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            wait_vmcnt<NPA + NPS>();   // every fetch into LDS has landed; only the prefetch is in flight
        } else {
#pragma unroll
            for (int q = 0; q < NPA + NPS; ++q) pf[q] = 0;
            wait_vmcnt<0>();   // nothing may still be landing in LDS once it holds the output
        }
    }

    store_tile<PATH, WM, WN, TM, TN, BIAS, OUT, ((B4 || A4 || F6) ? BODY : OPND_BYTES), PRM>(p, acc, &lds[0], &lds[PRM_OFF], m0, n0,
                                                                            rows_a, rows_b);
    // (the prefetched values, consumed here so that the loads stay: the wait
    // for them falls after the output stores)
    if constexpr (SUCC) {
#pragma unroll
        for (int q = 0; q < NPA + NPS; ++q)
            asm volatile("" : : "v"(pf[q]));
    }
}

}  // namespace qgemm
