// fl_dma16.hpp -- the fused GEMM with direct-to-LDS loads: fp16/bf16 (or
// FP8 E4M3) operands, fp32 accumulation, the fused epilogue.
//
// Same contract and epilogue as FusedTile (fl_kernels.hpp); this variant
// serves every fp16/bf16 and FP8-operand problem.  Pointers need only
// element alignment: 16-byte buffer loads and the 8-byte epilogue accesses
// may be unaligned on gfx950.  With N % 8 != 0 (16 for FP8 codes) a B chunk
// that crosses N brings in the next row's first values, which only reach
// output columns >= N (never stored); with K % 8 != 0 (16) the straddling A
// chunk is masked in LDS (fix_k_tail) and B's rows >= K are read as zeros.
// Differences from the register-staged kernel:
//
//   * Global -> LDS copies use buffer_load_dwordx4 with the LDS bit: each
//     instruction moves 64 x 16 bytes straight into 1 KB of LDS at
//     M0 + lane*16, so no staging registers, no ds_write and no VALU
//     transposes.  The XOR swizzle is applied on the global side: lane l of
//     an instruction fetches the chunk that belongs at LDS position l.
//   * B stays N-contiguous in LDS ([k][n] rows) and its MFMA operand is read
//     with ds_read_b64_tr_b16 (or _tr_b8 for FP8): within each 16-lane
//     group, lane i receives element 16*j + i (j = 0..3) of the group's
//     lane-major 64 values, so 16 lanes that point at 4 k-rows x 16 columns
//     (4 columns per lane) receive one column each with 4 consecutive k
//     values -- the K-contiguous B operand of the MFMA.
//   * A K stage of BK values (64 for 16-bit operands, 128 for FP8: A rows
//     are whole 128-byte lines; 32 or 64 where A rows are 64 bytes)
//     occupies one of NBUF LDS buffers.
//     The copies of a stage are issued right after the barrier that frees
//     its buffer, so NBUF-1 stages are in flight while MFMAs run
//     ("Optimizing GEMM + Activation on CDNA4 with TLX", "Version 3": a
//     deeper buffer ring lets the wait keep loads in flight instead of
//     draining them).
//   * Each stage is BK/KPM blocks of MFMAs; the operand reads of the next
//     block are slotted between the MFMAs of the current one, and the one
//     barrier per stage sits before the last block, whose MFMA slots also
//     carry the copies of the stage NBUF ahead.
//   * The copies are inline asm, invisible to the compiler's wait-count
//     pass; every wait on them is explicit (wait_vm).
#pragma once

#include "fl_kernels.hpp"

namespace fl {

#define FL_LDS __attribute__((address_space(3)))

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

// Buffer descriptor in SGPRs (gfx9 layout: 48-bit base, stride 0,
// num_records, word 3 = 32-bit data format) for the inline-asm copies.
__device__ __forceinline__ i32x4_t sgpr_rsrc(const void *p, size_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    const uint32_t n = bytes > 0x7fffffffull ? 0x7fffffffu : (uint32_t)bytes;
    i32x4_t r;
    r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
    r.z = __builtin_amdgcn_readfirstlane((int)n);
    r.w = (int)kRsrcWord3;
    return r;
}

// One 64 x 16-byte copy from global memory into LDS at lds_addr + lane*16
// (byte address base + soffset + voffset; a voffset at or past num_records
// writes zeros).  M0 is written here and used by nothing else in the
// kernels that call this.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(i32x4_t rsrc, uint32_t voffset, uint32_t soffset, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voffset), "s"(rsrc),
                 "s"(soffset), "s"(lds_addr)
                 : "memory", "m0");
}
// One 16-bit (or 8-bit) load and its wait in a single asm block.  A load into a VGPR
// that the compiler sees, issued on a branch inside the K loop, makes its
// wait-count pass assume the register may still be pending on every later
// pass through the loop, and it then drains all outstanding copies
// (vmcnt(0)) before the next LDS read into that register: the look-ahead
// copies would land in lock step with the MFMAs.  Hidden here, the only
// vector-memory operations the compiler tracks in the loop are none, and
// every wait on the copies is an explicit one.
__device__ __forceinline__ uint32_t load_u16_now(i32x4_t rsrc, uint32_t voffset) {
    uint32_t v;
    asm volatile("buffer_load_ushort %0, %1, %2, 0 offen\n\ts_waitcnt vmcnt(0)"
                 : "=&v"(v)
                 : "v"(voffset), "s"(rsrc)
                 : "memory");
    return v & 0xffffu;
}
__device__ __forceinline__ uint32_t load_u8_now(i32x4_t rsrc, uint32_t voffset) {
    uint32_t v;
    asm volatile("buffer_load_ubyte %0, %1, %2, 0 offen\n\ts_waitcnt vmcnt(0)"
                 : "=&v"(v)
                 : "v"(voffset), "s"(rsrc)
                 : "memory");
    return v & 0xffu;
}
#pragma clang diagnostic pop

// WAVES_N waves along N and 2 along M: 4 waves (one per SIMD, 128 x BN/2
// each) or 8 waves (two per SIMD, 128 x BN/4 each; the two waves sharing a
// SIMD own the same columns and cover each other's waits).  SPREAD: the
// copies of a look-ahead stage are issued over that many blocks (the block
// after the barrier that frees their buffer and the next SPREAD-1 blocks)
// instead of all in one, so the address unit's queue does not fill up and
// hold back the MFMAs behind them.  OCC: workgroups resident per CU; with 2
// the LDS ring and the epilogue staging fit in half of the LDS (72 KB) and
// the registers in half of the register file, so one workgroup's epilogue
// and start-up overlap the other's K loop.  RES: the epilogue adds the
// residual a.R (compiled in only where it is used, so the plain epilogue
// keeps its registers).  QF: -1 stores the I/O dtype; FL_Q_FP8_E4M3 or
// FL_Q_INT8 store one-byte codes of the epilogue value times a.scale.  IN:
// the type of A and B, DT (fp16/bf16) or kInFp8 (OCP E4M3 codes, fp8 MFMA,
// the accumulator scaled by a.ab_scale before the bias; bias, Y and out
// stay in DT).  BWD: the backward epilogue (see epilogue_lds), with B given
// as (N, K) row-major (the weight read as its transpose): its tile is
// staged and read exactly like A's, and a lane's 16-byte read of a row is
// already the MFMA's B fragment (8 consecutive k of one column).  M16:
// the product runs as 16x16 output blocks 32 deep (v_mfma_f32_16x16x32_
// {f16,bf16}; FP8: 16x16x128) instead of 32x32 blocks 16 deep (32x32x64);
// same flops per operand read from LDS for the wave's tile, but on random
// data the matrix cores hold a higher clock under the 16x16 form (measured
// with operands in registers: 1838 against 1645 TFLOP/s, 2.29 against 2.01
// GHz, 8 waves per CU).
template <int DT, int ACT, int BK_, int BN_ = 256, int WAVES_N = 2, int SPREAD = 1, int OCC = 1, bool RES = false,
          int QF = -1, int IN = DT, bool BWD = false, bool M16 = false>
struct Dma16 {
    using base = FusedTile<DT, ACT, true>;  // shares the epilogue
    static constexpr bool F8 = IN == kInFp8;
    static constexpr bool BT = BWD;  // B is (N, K) row-major, K contiguous
    static constexpr int IES = F8 ? 1 : 2;           // bytes per A/B element
    static constexpr int EPCH = 16 / IES;            // A/B elements per 16-byte chunk
    static constexpr int KPM = F8 ? (M16 ? 128 : 64) : M16 ? 32 : 16;  // K per MFMA: 16x16x128 / 32x32x64 fp8,
                                                                        // 16x16x32 / 32x32x16 16-bit
    static constexpr int BM = 256, BN = BN_, BK = BK_;
    static_assert(BK * IES == 64 || BK * IES == 128, "stage depth: 64- or 128-byte A rows");
    static_assert(BN == 128 || BN == 192 || BN == 256, "tile width");
    static_assert(WAVES_N == 2 || WAVES_N == 4, "wave grid");
    static_assert(BN % ((M16 ? 16 : 32) * WAVES_N) == 0, "whole MFMA blocks per wave");
    static_assert(BN != 192 || !F8 || !M16, "the 192-wide FP8 swizzle is for 32x32x64 blocks");
    static constexpr int WAVES = 2 * WAVES_N, THREADS = 64 * WAVES;
    static constexpr int WN = BN / WAVES_N;          // wave tile: 128 x WN
    static constexpr int RBH = M16 ? 16 : 32;        // output rows of an accumulator block
    static constexpr int NRB = 128 / RBH;            // accumulator blocks per wave along M
    static constexpr int NI = WN / RBH;              // MFMA blocks per wave along N (square blocks)
    static constexpr int AV = M16 ? 4 : 16;          // accumulator floats per lane and block
    typedef float acc_t __attribute__((ext_vector_type(AV)));
    static constexpr int KK = BK / KPM;              // MFMA blocks per stage
    static constexpr int CA = BK * IES / 16;         // 16-byte chunks per A row
    static constexpr int CB = BN * IES / 16;         // 16-byte chunks per B row
    static constexpr int A_BYTES = BM * BK * IES;    // rows of BK*IES bytes
    static constexpr int B_BYTES = BK * BN * IES;    // rows of BN*IES bytes
    static constexpr int BUF_BYTES = A_BYTES + B_BYTES;
    static constexpr int LDS_RING = OCC == 2 ? 73728 : M16 ? 163840 : BN == 256 ? 131072 : BN == 128 ? 147456 : 163840;
    static constexpr int NBUF = LDS_RING / BUF_BYTES;  // LDS ring
    static constexpr int A_ROWS_PER_COPY = 64 / CA;  // A rows per 1 KB copy
    static constexpr int NA = BM / (A_ROWS_PER_COPY * WAVES);  // A copies per wave per stage
    // B: copy j of a stage covers its 16-byte chunks 64j .. 64j+63 in row
    // order (a copy may start and end inside a row when a row is not a
    // divisor of 1 KB).  The lane -> (row offset, chunk) pattern and the
    // swizzle repeat every PB copies, which span B_ROWS_PER_PERIOD rows (a
    // multiple of the swizzle's period in rows, FBP).
    // With 16x16 blocks the swizzle also depends on bit 3 of the row (period
    // 16 rows), which the copies of one wave need not repeat: each of them
    // keeps its own offset (PB = NB).
    static constexpr int FBP = F8 ? 8 : 4;
    static constexpr int pb_of(int p) { return ((64 * p) % CB == 0 && ((64 * p) / CB) % FBP == 0) ? p : pb_of(p + 1); }
    static constexpr int NB = BK * CB / (64 * WAVES);  // B copies per wave per stage
    static constexpr int PB = M16 ? NB : pb_of(2);     // 2 for every power-of-two width
    static constexpr int B_ROWS_PER_PERIOD = 64 * PB / CB;
    static constexpr int B_ROWS_PER_COPY_T = 64 / CA;  // K-contiguous B: its rows per 1 KB copy
    static constexpr int DMA_PER_WAVE = NA + NB;
    static constexpr int SLOTS = NRB * NI;           // MFMAs per block
    static constexpr int RPA = F8 ? 2 : 1;           // LDS reads per A operand (16 bytes each)
    static constexpr int RPB = F8 ? 4 : BT ? 1 : 2;  // reads per B operand (transposed 8-byte, or one 16-byte)
    static constexpr int BPARTS = F8 ? 4 : 2;        // 8-byte parts of a B operand
    static constexpr int READS = NRB * RPA + NI * RPB;  // operand reads per block
    static_assert(NA * WAVES * A_ROWS_PER_COPY == BM, "A copies cover the tile");
    static_assert(NB * WAVES * 64 == BK * CB, "B copies cover the stage");
    static_assert(NB % PB == 0, "each wave's first B copy starts a swizzle period");
    static_assert(!BT || (NB * WAVES * B_ROWS_PER_COPY_T == BN && NB % 2 == 0 && !F8 && QF < 0 && !RES),
                  "K-contiguous B: A-like copies with period 2; 16-bit operands, plain output");
    // The swizzle of an A copy's rows repeats with period 2 in the copy
    // index (Lane below keeps two offsets and a stride), so each wave's
    // first copy must have an even index: an even number of copies per wave.
    static_assert(NA % 2 == 0, "A copies per wave");
    // The copies of a stage are spread over SPR blocks (at most the blocks of
    // one stage).  With 16x16 blocks a stage has only two blocks (64 deep) or
    // one (32 deep), and all its copies go out in the block after the
    // barrier that frees their buffer: the copies of the second half would
    // otherwise have half a stage less to land (measured 1219 -> 1279
    // TFLOP/s at 4096^3 together with the read placement below).  FP8
    // stages take half the MFMA time of 16-bit ones, and the 256- and
    // 192-wide FP8 kernels issue their copies in one block too (+3% at
    // 4096^3, +7% on 1024x21568x4096); the 256x128 one, with three
    // buffers, keeps two (-2% in one).
    static constexpr int SPR = (M16 || (F8 && BN != 128)) ? 1 : SPREAD < KK ? SPREAD : KK;
    static_assert(SPREAD >= 1, "copies spread over one block at least");
    // Copies [part_lo(p), part_lo(p+1)) of a stage form part p.
    static constexpr int part_lo(int p) { return p * DMA_PER_WAVE / SPR; }
    static_assert(NBUF >= 2, "double buffering at least");
    static_assert(OCC == 1 || (OCC == 2 && WAVES == 4), "two resident workgroups of 4 waves");

    // A swizzle: chunk c of row r sits at c ^ fa(r).  16-byte operand reads
    // of 8 consecutive rows (8 lanes per cycle) and of 16 consecutive rows
    // (16 lanes per cycle) both touch distinct bank groups.
    __device__ __forceinline__ static int fa(int r) {
        if constexpr (CA == 4)
            return ((r >> 1) ^ (r >> 3)) & 3;
        else
            return ((r >> 1) ^ ((r & 1) << 2)) & 7;
    }
    // 16x16 blocks with 32-deep stages (64-byte A rows): each 16-row block
    // of the A stage is stored chunk-major, chunk c of row r at c*256 + r*16,
    // so that the operand read of a block (lane l: row l%16, chunk l/16) is
    // one linear 1 KB read, which the LDS serves without conflicts; 64-byte
    // rows read row-major cost twice the cycles whatever the chunk XOR
    // (measured).  A copy of 1 KB fills one such block: lane l fetches row
    // l%16, chunk l/16.
    static constexpr bool A_CM = M16 && CA == 4;
    __device__ __forceinline__ static int a_row_in_copy(int lane) { return A_CM ? (lane & 15) : lane / CA; }
    __device__ __forceinline__ static int a_chunk_in_copy(int lane, int r) {
        return A_CM ? (lane >> 4) : (lane % CA) ^ fa(r);
    }

    // B swizzle: chunk c of k-row r sits at c ^ fb(r).  16-bit B: fb in
    // {0,6,12,10} by r % 4 (rows are 256 or 512 bytes, a multiple of the bank
    // width); conflict-free for the transposed 8-byte reads (4 rows x 2 or 4
    // chunks per 16 or 32 lanes).
    //
    // FP8 B: a transposed 8-byte read serves 32 lanes per cycle, which touch
    // 8 k-rows in two 16-byte chunks each (32x32x64 blocks: chunks c and c+1,
    // c even) or in one chunk of 16 k-rows (16x16x128 blocks: rows 0..7 and
    // 32..39 of a 64-row group).  256-byte rows (BN = 256) span the 64 banks,
    // so the 16 (row, chunk) pairs need 16 different chunks: fb = 2*(r % 8)
    // puts chunk c of rows 0..7 on the 8 chunks of c's parity, and the XOR
    // of 1 by bit 5 of the row moves rows 32..63 to the other parity.
    // 128-byte rows (BN = 128) alternate between the two halves of the banks,
    // so fb = r % 8 (with the same bit-5 term) suffices: 4 rows of each half
    // x 2 chunks, or 8 rows of each half x 1 chunk, on 8 different chunks.
    // 192-byte rows (BN = 192, 32x32x64 blocks only): row r starts 12*r
    // chunk widths into the banks, so rows 0..3 start on the four quarters
    // of the bank width and rows 4..7 again on the same ones; fb = 2 on rows
    // 4..7 of every 8 moves their chunk pair (c, c+1) onto the other pair of
    // its aligned group of four (an XOR below 4 keeps every chunk inside its
    // row of 12), which leaves the 16 (row, chunk) pairs on 16 bank groups.
    //
    // 16-bit B, BN = 192: rows of 384 bytes, so odd rows already start half
    // a bank width (128 bytes) over; fb = r & 2 moves rows 2 and 3 of every
    // four by two chunks, which again leaves the 4 rows x 2 chunks of a
    // transposed read in 8 different bank groups.  An XOR below 8 keeps
    // every chunk inside its row of 24.
    //
    // 16x16 blocks: the four 16-lane groups of a transposed read take k-rows
    // 8 apart (rows g*8 + 0..3 of the same 16 columns), and two of them are
    // served in the same cycle; the XOR term from bit 3 of the row moves
    // rows 8..15 of every 16 by 2 chunks (4 for 192-wide rows), into the
    // bank groups rows 0..7 leave free.
    __device__ __forceinline__ static int fb(int r) {
        if constexpr (F8 && BN == 192)
            return (r >> 1) & 2;
        else if constexpr (F8)
            return (BN == 256 ? (r & 7) << 1 : (r & 7)) ^ (M16 ? ((r >> 5) & 1) : 0);
        else if constexpr (BN == 192)
            return (r & 2) ^ (M16 ? ((r >> 1) & 4) : 0);
        else
            return ((0xAC60 >> (4 * (r & 3))) & 0xF) ^ (M16 ? ((r >> 2) & 2) : 0);
    }

    // Per-lane copy offsets and operand-read addresses, fixed for a tile.
    // A is addressed through a descriptor based at row m0 and B through one
    // based at column n0; a stage adds its K origin as the scalar offset
    // (k0*2 bytes for A, k0*N*2 for B).  A lane whose chunk lies past K (or
    // past N) uses kOob so the hardware range check writes zeros; rows past
    // M are beyond num_records of A's descriptor.  Copy i of a wave covers
    // A rows A_ROWS_PER_COPY*(wave*NA + i) + lane/CA, whose swizzle repeats
    // with period 2 in i, and B stage chunk 64*(wave*NB + i) + lane, whose
    // row offset and swizzle repeat with period PB; so PB + 2 offsets and
    // two strides describe all copies.
    struct Lane {
        i32x4_t rA, rB;
        uint32_t a_off[2];  // byte offset (k0 = 0) of copies i = 0, 1; +i/2 * a_step
        int a_k[2];         // K index within the stage of those chunks
        uint32_t b_off[PB]; // same for B (kOob when the columns are past N); +i/PB * b_step
        int b_kr[PB];       // K row within the stage of copies i = 0..PB-1 (+i/PB * B_ROWS_PER_PERIOD)
        int b_k[2];         // K-contiguous B: K index within the stage of copies 0, 1 (as a_k)
        uint32_t a_step, b_step;
        int a_frag[KK];     // LDS byte address of A operand reads per kk (mi adds 32 rows)
        int b_frag[BT ? KK : NI];  // B operand reads per ni (kk adds 16 rows, h 4 rows); per kk when K-contiguous
    };

    __device__ __forceinline__ static void setup(const GemmArgs &a, int m0, int n0, int wave, int lane, int wm,
                                                 int wn, Lane &L) {
        const size_t a_org = (size_t)m0 * a.K;
        L.rA = sgpr_rsrc(static_cast<const char *>(a.A) + a_org * IES, ((size_t)a.M * a.K - a_org) * IES);
        if constexpr (BT)
            L.rB = sgpr_rsrc(static_cast<const char *>(a.B) + (size_t)n0 * a.K * IES,
                             ((size_t)a.N * a.K - (size_t)n0 * a.K) * IES);
        else
            L.rB = sgpr_rsrc(static_cast<const char *>(a.B) + (size_t)n0 * IES, ((size_t)a.K * a.N - n0) * IES);
#pragma unroll
        for (int i = 0; i < (PB > 2 ? PB : 2); ++i) {
            if (i < 2) {
                const int ra = A_ROWS_PER_COPY * (wave * NA + i) + a_row_in_copy(lane);
                const int ca = a_chunk_in_copy(lane, ra);
                L.a_off[i] = (uint32_t)(ra * a.K + ca * EPCH) * IES;
                L.a_k[i] = ca * EPCH;
            }
            if (BT && i < 2) {
                // as A: rows of B^T (output columns), chunks along K
                const int rb = B_ROWS_PER_COPY_T * (wave * NB + i) + lane / CA;
                const int cb = (lane % CA) ^ fa(rb);
                L.b_off[i] = (uint32_t)(rb * a.K + cb * EPCH) * IES;
                L.b_k[i] = cb * EPCH;
            }
            if (!BT && i < PB) {
                // chunk q of the stage in row order: row q / CB, chunk q % CB
                const int q = 64 * (wave * NB + i) + lane;
                const int rb = (64 % CB == 0) ? (64 / CB) * (wave * NB + i) + lane / CB : q / CB;
                const int cb = ((64 % CB == 0) ? lane % CB : q % CB) ^ fb(rb);
                L.b_off[i] = (n0 + cb * EPCH < a.N) ? (uint32_t)(rb * a.N + cb * EPCH) * IES : kOob;
                L.b_kr[i] = rb;
            }
        }
        L.a_step = (uint32_t)(2 * A_ROWS_PER_COPY * a.K) * IES;
        L.b_step = BT ? (uint32_t)(2 * B_ROWS_PER_COPY_T * a.K) * IES : (uint32_t)(B_ROWS_PER_PERIOD * a.N) * IES;
        const int lrow = lane & 31, lg = lane >> 5;
        const int r = wm * 128 + lrow;
        const int g16 = lane >> 4, i16 = lane & 15;
        if constexpr (BT) {
            // rows of the B^T tile are output columns; fa depends on the row
            // modulo 16 only, so one address per kk serves every ni (+32 rows,
            // or +16 with 16x16 blocks, whose lanes take chunk kk*4 + g16 of
            // rows i16 as the A operand does)
            const int rA = M16 ? wm * 128 + i16 : r;
            const int rn = wn * WN + (M16 ? i16 : lrow);
            const int ck = M16 ? g16 : lg, kst = M16 ? 4 : 2;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                L.a_frag[kk] = rA * (BK * 2) + (((kk * kst + ck) ^ fa(rA)) * 16);
                L.b_frag[kk] = A_BYTES + rn * (BK * 2) + (((kk * kst + ck) ^ fa(rn)) * 16);
            }
        } else if constexpr (F8 && M16) {
            // FP8 in 16x16 blocks 128 deep (v_mfma_scale_f32_16x16x128):
            // A: lane (row i16, group g16) takes k = g16*32 .. g16*32+31 of
            // the block, chunks kk*8 + g16*2 and the next one (address bit 4).
            const int r16 = wm * 128 + i16;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) L.a_frag[kk] = r16 * (BK * IES) + (((kk * 8 + g16 * 2) ^ fa(r16)) * 16);
            // B: lane L of group g16 points at k-row g16*32 + L/2 (+8 per
            // transposed read), 8 columns at 8*(L%2) of the 16-column block:
            // it then holds 8 k-values of column i16 per read.
            const int rk = g16 * 32 + (i16 >> 1);
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                const int n = wn * WN + ni * 16 + 8 * (i16 & 1);
                L.b_frag[ni] = A_BYTES + rk * BN + (((n >> 4) ^ fb(rk)) * 16) + (n & 15);
            }
        } else if constexpr (M16) {
            // A: lane (row r16, group g16) takes k = g16*8 .. g16*8+7 of each
            // 32-deep block: chunk kk*4 + g16; fa depends on the row modulo
            // 16 only, so blocks mi > 0 add 16 rows to this address.
            const int r16 = wm * 128 + i16;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                L.a_frag[kk] = A_CM ? wm * 128 * (BK * 2) + g16 * 256 + i16 * 16
                                    : r16 * (BK * 2) + (((kk * 4 + g16) ^ fa(r16)) * 16);
            // B: 16-lane group g16 covers k-rows g16*8 .. g16*8+7 of the block
            // in two transposed reads (h adds 4 rows); lane i16 points at k-row
            // i16/4 of the four and at columns 4*(i16%4) .. +3 of the 16.
            const int rk = g16 * 8 + (i16 >> 2);
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                const int n = wn * WN + ni * 16 + 4 * (i16 & 3);
                L.b_frag[ni] = A_BYTES + rk * (BN * 2) + (((n >> 3) ^ fb(rk)) * 16) + ((n >> 2) & 1) * 8;
            }
        } else if constexpr (!F8) {
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) L.a_frag[kk] = r * (BK * 2) + (((kk * 2 + lg) ^ fa(r)) * 16);
            const int rk = (g16 >> 1) * 8 + (i16 >> 2);  // k-row for kk = 0, h = 0
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                const int n = wn * WN + ni * 32 + (g16 & 1) * 16 + 4 * (i16 & 3);
                L.b_frag[ni] = A_BYTES + rk * (BN * 2) + (((n >> 3) ^ fb(rk)) * 16) + ((n >> 2) & 1) * 8;
            }
        } else {
            // A: lane (row r, half lg) takes k = lg*32 .. lg*32+31 of each
            // 64-deep block: chunks kk*4 + lg*2 and the next one, whose
            // swizzled address differs in bit 4 (c even: (c+1)^f = (c^f)^1).
            // The fp8 MFMA pairs byte j of lane half lg in both operands, so
            // any k order works if A and B use the same one.
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) L.a_frag[kk] = r * (BK * IES) + (((kk * 4 + lg * 2) ^ fa(r)) * 16);
            // B: a 16-lane transposed read gives lane i byte i%8 from lanes
            // i/8 + 2j (j = 0..7), so lane L of group g16 points at k-row
            // lg*32 + L/2 (+8 per read t), 8 columns at 8*(L%2): the lane
            // then holds 8 k-values of column (g16 & 1)*16 + i16.
            const int rk = lg * 32 + (i16 >> 1);
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                const int n = wn * WN + ni * 32 + (g16 & 1) * 16 + 8 * (i16 & 1);
                L.b_frag[ni] = A_BYTES + rk * BN + (((n >> 4) ^ fb(rk)) * 16) + (n & 15);
            }
        }
    }

    // K row within the stage of this lane's chunk of B copy i.
    __device__ __forceinline__ static int b_row(const Lane &L, int i) {
        if constexpr (64 % CB == 0)
            return L.b_kr[0] + (64 / CB) * i;
        else
            return L.b_kr[i % PB] + B_ROWS_PER_PERIOD * (i / PB);
    }

    struct Stage {  // scalar state of the copies of one stage
        int kleft;
        uint32_t soa, sob;
        uint32_t adst, bdst;  // LDS byte address of this wave's first A / B copy
    };

    __device__ __forceinline__ static Stage stage_of(const GemmArgs &a, int kt, int wave, uint32_t buf_addr) {
        const int k0 = kt * BK;
        Stage s;
        s.kleft = a.K - k0;
        s.soa = (uint32_t)k0 * IES;
        s.sob = BT ? (uint32_t)k0 * IES : (uint32_t)k0 * (uint32_t)a.N * IES;
        s.adst = __builtin_amdgcn_readfirstlane(buf_addr + wave * NA * 1024);
        s.bdst = __builtin_amdgcn_readfirstlane(buf_addr + A_BYTES + wave * NB * 1024);
        return s;
    }

    // Copy I (A copies first) of the stage described by s.  Stages at or past
    // the end of K are issued too, with every lane out of range, so every
    // stage issues the same number of copies and the wait counts are
    // constants.
    template <int I>
    __device__ __forceinline__ static void copy_one(const Lane &L, const Stage &s) {
        if constexpr (I < NA) {
            const uint32_t off = L.a_off[I & 1] + (uint32_t)(I >> 1) * L.a_step;
            lds_copy16(L.rA, L.a_k[I & 1] < s.kleft ? off : kOob, s.soa, s.adst + I * 1024);
        } else if constexpr (BT) {
            constexpr int i = I - NA;
            const uint32_t off = L.b_off[i & 1] + (uint32_t)(i >> 1) * L.b_step;
            lds_copy16(L.rB, L.b_k[i & 1] < s.kleft ? off : kOob, s.sob, s.bdst + i * 1024);
        } else {
            constexpr int i = I - NA;
            const uint32_t off = L.b_off[i % PB] + (uint32_t)(i / PB) * L.b_step;
            const bool ok = (b_row(L, i) < s.kleft) && (L.b_off[i % PB] != kOob);
            lds_copy16(L.rB, ok ? off : kOob, s.sob, s.bdst + i * 1024);
        }
    }

    template <int I = 0>
    __device__ __forceinline__ static void copy_all(const Lane &L, const Stage &s) {
        if constexpr (I < DMA_PER_WAVE) {
            copy_one<I>(L, s);
            copy_all<I + 1>(L, s);
        }
    }

    // Fix-up of the last K stage (origin kt*BK) when K or N is not a
    // multiple of EPCH (the elements of a 16-byte chunk), run by each wave on
    // the chunks it copied, after its copies have landed and before the
    // barrier that publishes them:
    //  * an A chunk that straddles K also holds the first values of the next
    //    row; the values at or past K are zeroed so that only k < K reaches
    //    the accumulators (B's rows at or past K read as zeros);
    //  * a copy that runs past the end of A (or B) is range-checked per
    //    dword, so a dword that holds the buffer's last bytes and runs past
    //    it reads as zero: with 2-byte elements the last element, with FP8
    //    codes up to the last three.  A lane whose chunk holds one of those
    //    elements (one that belongs to its own row, below K, or below N for
    //    B) reloads it with a 1- or 2-byte load and writes it into LDS.  The
    //    reload goes through the tile's own descriptor (based at row m0 of A,
    //    at column n0 of B, or at row n0 of the transposed B), so its offset
    //    is below 256 rows of the operand, which the host keeps under 2^31
    //    bytes, however large the whole operand is.  The elements a partial
    //    dword can hold lie in the last row of B (the host asks for N >= 3
    //    with FP8 codes), so the last stage has them.
    static constexpr int EPD = 4 / IES;  // elements per dword

    __device__ __forceinline__ static uint32_t keep_mask(int valid, int d) {
        const int vb = valid * IES - 4 * d;  // bytes of dword d below the end of the row
        return vb >= 4 ? 0xffffffffu : vb <= 0 ? 0u : (1u << (8 * vb)) - 1u;
    }

    __device__ __forceinline__ static uint32_t load_elem_now(i32x4_t rsrc, uint32_t voffset) {
        if constexpr (F8)
            return load_u8_now(rsrc, voffset);
        else
            return load_u16_now(rsrc, voffset);
    }

    // Reload the elements of a chunk that a partial last dword may have
    // zeroed: elements e = first .. valid-1 (at most EPD-1 of them), element
    // e at byte offset (rel + e) * IES of the descriptor.  All in 32 bits:
    // the offsets stay below 256 rows (A, B^T) or below the whole operand
    // (B), which the host keeps under 2^31 bytes.
    __device__ __forceinline__ static void reload_one(i32x4_t rsrc, uint32_t rel, int e, u32x4_t &v) {
        const uint32_t x = load_elem_now(rsrc, (rel + e) * IES);
        const int sh = 8 * ((e * IES) & 3);
        const uint32_t m = (F8 ? 0xffu : 0xffffu) << sh;
        v[(e * IES) >> 2] = (v[(e * IES) >> 2] & ~m) | (x << sh);
    }
    __device__ __forceinline__ static void reload_tail(i32x4_t rsrc, uint32_t rel, int first, int valid, u32x4_t &v) {
        if constexpr (EPD == 2) {
            // 2-byte elements: the one element `first` (>= 0 where called)
            if (first < valid) reload_one(rsrc, rel, first, v);
        } else {
            for (int e = first > 0 ? first : 0; e < valid; ++e) reload_one(rsrc, rel, e, v);
        }
    }

    // The K-contiguous operand (A, or B^T): chunk of row `row` (of `rows`,
    // the descriptor based at row `r0`) starting at k = kc, `valid` values
    // below K.  Only the last EPD-1 rows can hold an element of the
    // buffer's last dword.
    __device__ __forceinline__ static void fix_kc_chunk(i32x4_t rsrc, int row, int rows, int r0, int K, int kc,
                                                        int valid, FL_LDS char *p) {
        u32x4_t v = *(FL_LDS u32x4_t *)p;
#pragma unroll
        for (int d = 0; d < 4; ++d) v[d] &= keep_mask(valid, d);
        const int dr = rows - row;  // 1 for the last row
        if (dr > 0 && dr < EPD)
            reload_tail(rsrc, (uint32_t)((row - r0) * K + kc), dr * K - (EPD - 1) - kc, valid, v);
        *(FL_LDS u32x4_t *)p = v;
    }

    __device__ __forceinline__ static void fix_k_tail(const GemmArgs &a, const Lane &L, int m0, int n0, int kt,
                                                      int wave, int lane, FL_LDS char *buf) {
        const int k0 = kt * BK, kleft = a.K - k0;
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int kb = L.a_k[i & 1];
            const int valid = kleft - kb;  // values of this chunk below K
            if (valid > 0 && valid < EPCH)
                fix_kc_chunk(L.rA, m0 + A_ROWS_PER_COPY * (wave * NA + i) + a_row_in_copy(lane), a.M, m0, a.K,
                             k0 + kb, valid, buf + (wave * NA + i) * 1024 + lane * 16);
        }
        if constexpr (BT) {
            // B^T rows are K-contiguous like A's: the same two fixes
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int kb = L.b_k[i & 1];
                const int valid = kleft - kb;
                if (valid > 0 && valid < EPCH)
                    fix_kc_chunk(L.rB, n0 + B_ROWS_PER_COPY_T * (wave * NB + i) + lane / CA, a.N, n0, a.K, k0 + kb,
                                 valid, buf + A_BYTES + (wave * NB + i) * 1024 + lane * 16);
            }
        } else if (a.N % EPCH) {
            // columns at or past N are never stored, so only the reload, of
            // elements of B's last row (N >= EPD-1 where FP8 codes are read)
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int rb = b_row(L, i);  // K row within the stage
                const int cb = ((64 % CB == 0) ? lane % CB : (64 * (wave * NB + i) + lane) % CB) ^ fb(rb);
                const int col = n0 + cb * EPCH;
                const int vn = a.N - col < EPCH ? a.N - col : EPCH;  // values of this chunk below N
                const int first = a.N - (EPD - 1) - col;              // chunk element of the first reload
                if (rb == kleft - 1 && vn > 0 && first < vn) {
                    FL_LDS char *p = buf + A_BYTES + (wave * NB + i) * 1024 + lane * 16;
                    u32x4_t v = *(FL_LDS u32x4_t *)p;
                    reload_tail(L.rB, (uint32_t)((a.K - 1) * a.N + (col - n0)), first, vn, v);
                    *(FL_LDS u32x4_t *)p = v;
                }
            }
        }
    }

    struct Frags {
        u32x4_t a[NRB][RPA];   // A operand per mi (16 bytes per read)
        i32x2_t b[NI][BPARTS]; // B operand per ni (8 bytes per transposed read, or halves of one 16-byte read)
    };

    // Operand read number P of the READS that make up one kk block, in the
    // order the MFMAs of a block consume them: a0, b0 (RPB pieces) ..
    // b(NI-1), a1..a3 (RPA pieces each).
    template <int P>
    __device__ __forceinline__ static void read_piece(const Lane &L, const FL_LDS char *buf, int kk, Frags &f) {
        if constexpr (P < RPA) {
            f.a[0][P] = *(const FL_LDS u32x4_t *)(buf + (L.a_frag[kk] ^ (P * 16)));
        } else if constexpr (P < RPA + NI * RPB) {
            constexpr int ni = (P - RPA) / RPB, h = (P - RPA) % RPB;
            if constexpr (BT) {
                const u32x4_t v = *(const FL_LDS u32x4_t *)(buf + L.b_frag[kk] + ni * RBH * (BK * 2));
                f.b[ni][0] = i32x2_t{(int)v[0], (int)v[1]};
                f.b[ni][1] = i32x2_t{(int)v[2], (int)v[3]};
            } else if constexpr (!F8)
                f.b[ni][h] = __builtin_bit_cast(i32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                             (FL_LDS s16x4_t *)(buf + L.b_frag[ni] + kk * KPM * (BN * 2) +
                                                                                h * 4 * (BN * 2))));
            else
                f.b[ni][h] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (FL_LDS i32x2_t *)(buf + L.b_frag[ni] + kk * KPM * BN + h * 8 * BN));
        } else {
            constexpr int Q = P - RPA - NI * RPB;
            constexpr int mi = 1 + Q / RPA, h = Q % RPA;
            f.a[mi][h] = *(const FL_LDS u32x4_t *)(buf + ((L.a_frag[kk] + mi * RBH * BK * IES) ^ (h * 16)));
        }
    }

    template <int P = 0>
    __device__ __forceinline__ static void read_all(const Lane &L, const FL_LDS char *buf, int kk, Frags &f) {
        if constexpr (P < READS) {
            read_piece<P>(L, buf, kk, f);
            read_all<P + 1>(L, buf, kk, f);
        }
    }
    template <int P0, int P1>
    __device__ __forceinline__ static void read_range(const Lane &L, const FL_LDS char *buf, int kk, Frags &f) {
        if constexpr (P0 < P1) {
            read_piece<P0>(L, buf, kk, f);
            read_range<P0 + 1, P1>(L, buf, kk, f);
        }
    }

    // MFMA I of a block.  16x16 blocks and FP8 run the rows of blocks in
    // snake order (odd rows right to left), so that consecutive MFMAs always
    // share one operand: fewer operand bits toggle, which lowers the matrix
    // cores' power and lets the chip hold a higher clock (+1-2% measured
    // with 16x16 blocks, +0.5% with FP8).  The order of the MFMAs of one
    // output block, and so every result bit, is unchanged.
    template <int I>
    __device__ __forceinline__ static void mma_one(const Frags &f, acc_t (&acc)[NRB][NI]) {
        constexpr int mi = I / NI, ni = ((M16 || F8) && (mi & 1)) ? NI - 1 - I % NI : I % NI;
        if constexpr (F8) {
            const i32x4_t b01 = __builtin_shufflevector(f.b[ni][0], f.b[ni][1], 0, 1, 2, 3);
            const i32x4_t b23 = __builtin_shufflevector(f.b[ni][2], f.b[ni][3], 0, 1, 2, 3);
            const i32x8_t bv = __builtin_shufflevector(b01, b23, 0, 1, 2, 3, 4, 5, 6, 7);
            const i32x8_t av = __builtin_shufflevector(__builtin_bit_cast(i32x4_t, f.a[mi][0]),
                                                       __builtin_bit_cast(i32x4_t, f.a[mi][1]), 0, 1, 2, 3, 4, 5, 6, 7);
            // format codes 0, 0: both operands FP8 E4M3; no block scales
            if constexpr (M16)
                acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bv, av, acc[mi][ni], 0, 0, 0, 0, 0, 0);
            else
                acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bv, av, acc[mi][ni], 0, 0, 0, 0, 0, 0);
            return;
        }
        const s16x8_t bv = __builtin_bit_cast(
            s16x8_t, __builtin_shufflevector(f.b[ni][0], f.b[ni][1], 0, 1, 2, 3));
        if constexpr (M16) {
            if constexpr (DT == FL_F16)
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, bv),
                                                                     __builtin_bit_cast(f16x8_t, f.a[mi][0]),
                                                                     acc[mi][ni], 0, 0, 0);
            else
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, bv),
                                                                      __builtin_bit_cast(bf16x8_t, f.a[mi][0]),
                                                                      acc[mi][ni], 0, 0, 0);
        } else if constexpr (DT == FL_F16) {
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, bv),
                                                                 __builtin_bit_cast(f16x8_t, f.a[mi][0]), acc[mi][ni],
                                                                 0, 0, 0);
        } else {
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, bv),
                                                                  __builtin_bit_cast(bf16x8_t, f.a[mi][0]),
                                                                  acc[mi][ni], 0, 0, 0);
        }
    }

    // Copies [C0, C1) of a look-ahead stage.
    template <int C0, int C1>
    __device__ __forceinline__ static void copy_range(const Lane &L, const Stage &s) {
        if constexpr (C0 < C1) {
            copy_one<C0>(L, s);
            copy_range<C0 + 1, C1>(L, s);
        }
    }

    // One block: the SLOTS MFMAs on `use`, with the READS operand reads of
    // block kk_next of buffer `src` (into `fill`) in the last READS slots
    // and copies [C0, C1) of the look-ahead stage `s` spread over all slots.
    // Without copies the reads follow the first MFMAs.  16x16 blocks spread
    // the reads evenly over the block instead: a wave's next operands are
    // then all requested well before the block ends.
    template <int I, int C0, int C1>
    __device__ __forceinline__ static void block(const Lane &L, const FL_LDS char *src, int kk_next, const Stage &s,
                                                 const Frags &use, Frags &fill, acc_t (&acc)[NRB][NI]) {
        if constexpr (I < SLOTS) {
            constexpr int NC = C1 - C0;
            mma_one<I>(use, acc);
            copy_range<C0 + (I * NC + SLOTS - 1) / SLOTS, C0 + ((I + 1) * NC + SLOTS - 1) / SLOTS>(L, s);
            if constexpr (M16) {
                read_range<I * READS / SLOTS, (I + 1) * READS / SLOTS>(L, src, kk_next, fill);
            } else if constexpr (READS <= SLOTS) {
                constexpr int R = NC > 0 ? I - (SLOTS - READS) : I;
                if constexpr (R >= 0 && R < READS) read_piece<R>(L, src, kk_next, fill);
            } else {
                read_range<I * READS / SLOTS, (I + 1) * READS / SLOTS>(L, src, kk_next, fill);
            }
            __builtin_amdgcn_sched_barrier(0);
            block<I + 1, C0, C1>(L, src, kk_next, s, use, fill, acc);
        }
    }

    // vmcnt(n) with expcnt/lgkmcnt left unconstrained (gfx9 encoding).  The
    // copies are invisible to the compiler, so the wait is also a compiler
    // memory barrier: no LDS access may be moved above it.
    template <int N>
    __device__ __forceinline__ static void wait_vm() {
        static_assert(N >= 0 && N < 64, "vmcnt range");
        __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
        asm volatile("" ::: "memory");
    }

    // Blocks J..KK-1 of stage kt, held in LDS buffer `buf` (uniform, kept
    // at run time so that one copy of the stage code serves every buffer and
    // every stage count: no unrolled group, no separate tail).  On entry the
    // operands of block J are in f[J & 1] and `pend` describes the
    // look-ahead stage whose part 0 of the copies was issued in the block
    // before this stage; blocks 0..SPREAD-2 issue its parts 1..SPREAD-1.
    // Before the last block: wait until this wave's copies of stage kt+1
    // have landed (those of stages kt+2 .. kt+NBUF-1, all issued by then,
    // stay in flight) and barrier, after which stage kt+1 is visible to
    // every wave and buffer `buf` has been read by all of them, so the last
    // block starts refilling it with stage kt+NBUF while reading stage
    // kt+1's first operands.
    // P: the operand buffer stage kt starts from (f[P]); with an odd number
    // of blocks per stage it alternates from one stage to the next.
    // TAIL: the stage may be the one before the last, which fixes up the
    // last stage's chunks (fix_k_tail).  With SPLIT_TAIL the K loop runs its
    // other stages from a copy without that code (the 8-wave loop of 64
    // MFMAs shrinks from about 500 instructions to 175).  The 4-wave kernels
    // with 16x16 blocks keep one loop: split, the compiler's allocation of
    // their 192 (or 128) accumulator registers rotates them through copies
    // (about 250 accumulator moves per pass), which the single loop avoids.
    static constexpr bool SPLIT_TAIL = !(M16 && WAVES == 4);
    template <int J = 0, int P = 0, bool TAIL = false>
    __device__ __forceinline__ static void stage(const GemmArgs &a, const Lane &L, const FL_LDS char *lds,
                                                 uint32_t lds_addr, int m0, int n0, int kt, int nk, int buf,
                                                 int wave, Stage &pend, Frags (&f)[2], acc_t (&acc)[NRB][NI]) {
        const FL_LDS char *cur = lds + buf * BUF_BYTES;
        if constexpr (J < KK - 1) {
            constexpr int p = J + 1 < SPR ? J + 1 : SPR;  // part SPR is empty
            block<0, part_lo(p), part_lo(p < SPR ? p + 1 : p)>(L, cur, J + 1, pend, f[(J + P) & 1],
                                                                f[(J + P + 1) & 1], acc);
            stage<J + 1, P, TAIL>(a, L, lds, lds_addr, m0, n0, kt, nk, buf, wave, pend, f, acc);
        } else {
            const int nbuf = buf + 1 == NBUF ? 0 : buf + 1;
            const FL_LDS char *nxt = lds + nbuf * BUF_BYTES;
            wait_vm<(NBUF - 2) * DMA_PER_WAVE>();
            if constexpr (TAIL)
                if (((a.K | a.N) % EPCH) && kt + 2 == nk)
                    fix_k_tail(a, L, m0, n0, kt + 1, wave, threadIdx.x & 63, (FL_LDS char *)nxt);
            __syncthreads();
            pend = stage_of(a, kt + NBUF, wave, lds_addr + buf * BUF_BYTES);
            block<0, 0, part_lo(1)>(L, nxt, 0, pend, f[(J + P) & 1], f[(J + P + 1) & 1], acc);
            if (a.debug_sync) {
                // the debugging schedule: every copy of this wave landed and
                // every wave here before the next stage begins
                wait_vm<0>();
                __syncthreads();
            }
        }
    }

    // The output is written once and not read again by this kernel: when
    // its rows start on 128-byte lines (a.stream_out), the stores carry the
    // non-temporal (streaming) policy bit, so the lines leave the L2 as they
    // are written instead of at the end-of-kernel write-back (measured +1% at
    // 4096^3, +2-3% on the 8192x14336 and gate shapes); on rows that are not
    // line-aligned the partial lines it then writes cost 10% (4097x3071).
    static constexpr int kStreamStore = 2;  // cache-policy operand: nt

    // --- epilogue through LDS ---
    // Phase 1 (registers): bias, activation and the one conversion, exactly
    // as FusedTile::epilogue computes them (same arithmetic, same order);
    // each lane writes its 4-value groups into LDS (rows padded to EPI_ROW
    // bytes so the 32 rows a write instruction touches fall in different
    // banks).  Phase 2: each lane reads 16 bytes of a row back and stores
    // them, so a store instruction writes whole 128-byte lines.  Where a
    // wave's slice of an output row is a whole number of lines, each wave
    // stages its 128 x WN tile in an area of its own and stores it; where it
    // is not (a 192-byte slice of a 384-byte row, or 64-byte slices of
    // one-byte codes), the waves stage the whole tile, meet at a barrier,
    // and each stores BM / WAVES whole tile rows, so no line is written in
    // two pieces by two waves.
    static constexpr int OES = QF < 0 ? 2 : 1;  // bytes per output element
    static constexpr bool SHARED_EPI = (WN * OES) % 128 != 0;
    static constexpr int EPI_ROW = (SHARED_EPI ? BN : WN) * OES + 16;
    static constexpr int EPI_WAVE = 128 * EPI_ROW;  // one wave's area (own-area layout)
    static constexpr int EPI_BYTES = SHARED_EPI ? BM * EPI_ROW : WAVES * EPI_WAVE;
    static_assert(EPI_BYTES <= (OCC == 2 ? 73728 : 163840), "epilogue staging fits in the workgroup's LDS");
    // A lane's accumulators form groups of 4 consecutive output columns of
    // one row: per accumulator row block (RBH rows), NG groups.  32x32
    // blocks: lane l holds row l%32 and, in block ni, columns ni*32 + q*8 +
    // (l/32)*4 + e (q, e = 0..3; group g = ni*4 + q).  16x16 blocks: lane l
    // holds row l%16 and columns ni*16 + (l/16)*4 + e (group g = ni).
    static constexpr int NG = M16 ? NI : 4 * NI;
    __device__ __forceinline__ static int gcol(int g, int lane) {  // column of group g within the wave's tile
        if constexpr (M16)
            return g * 16 + (lane >> 4) * 4;
        else
            return (g >> 2) * 32 + (g & 3) * 8 + (lane >> 5) * 4;
    }
    __device__ __forceinline__ static float accv(const acc_t (&acc)[NRB][NI], int mi, int g, int e) {
        if constexpr (M16)
            return acc[mi][g][e];
        else
            return acc[mi][g >> 2][(g & 3) * 4 + e];
    }
    // Backward: the lanes' fp32 column sums of dX meet in the wave's own LDS
    // area as 32 rows (one per lane row) of WN floats, padded like EPI_ROW.
    static constexpr int DB_ROW = WN * 4 + 16;
    static_assert(!BWD || (!SHARED_EPI && WN == 64 && 32 * DB_ROW <= EPI_WAVE),
                  "backward: own-area staging, one bias column per lane");

    // Side input of the epilogue staged through LDS: SIDE 1 = Y (gate), 2 =
    // R (residual, or the saved X of the backward epilogue), 0 = none (or
    // one-byte output codes, whose staging rows are too narrow for it).
    // When N % 8 == 0 (no 16-byte chunk of a row crosses N), the tile's side
    // input is copied straight into the output staging area, at the place
    // of each output element, with one direct-to-LDS load per 1 KB, all
    // issued as the epilogue starts and waited for once.  A lane then reads
    // its values there and overwrites them with its results.  Otherwise it
    // is loaded into registers, one row block ahead.  The gate uses this
    // path for Y, so a residual or saved X next to it stays in registers.
    static constexpr int SIDE = QF >= 0 ? 0 : ACT == FL_ACT_GLU ? 1 : (RES || BWD) ? 2 : 0;
    // The gate's backward has a second side input, the saved X: where a
    // second staging area fits beside the first (own-area layout, one
    // workgroup per CU), it is copied into that area in the same way.
    static constexpr bool SIDE2 = BWD && ACT == FL_ACT_GLU && !SHARED_EPI && OCC == 1 && 2 * EPI_BYTES <= 163840;
    static constexpr int SMEM_BYTES =
        NBUF * BUF_BYTES > (SIDE2 ? 2 : 1) * EPI_BYTES ? NBUF * BUF_BYTES : (SIDE2 ? 2 : 1) * EPI_BYTES;

    // This wave's part of the staging area: its own 128 x WN tile, or in
    // the shared layout a run of the tile's 1 KB copies (the tile's staged
    // rows are contiguous: BM * RC chunks, a whole number of copies; with 8
    // waves on 192-wide rows the runs are 12 or 13 copies long).  Rows are
    // EPI_ROW bytes: the data and one 16-byte pad chunk, which is filled
    // with zeros (lanes given kOob).  Rows past M and columns past N read
    // zeros.
    __device__ __forceinline__ static void stage_side(const GemmArgs &a, const void *src, int m0, int n0, int wave,
                                                      int wm, int wn, int lane, uint32_t lds_addr) {
        constexpr int RC = EPI_ROW / 16;  // 16-byte chunks per staged row, the last one padding
        constexpr int YW = SHARED_EPI ? BN : WN;
        static_assert(EPI_ROW % 16 == 0 && RC == YW / 8 + 1, "padded rows of whole chunks");
        const size_t o_org = (size_t)m0 * a.N + n0;
        const i32x4_t rS = sgpr_rsrc(src ? static_cast<const char *>(src) + o_org * 2 : nullptr,
                                     src ? ((size_t)a.M * a.N - o_org) * 2 : 0);
        if constexpr (SHARED_EPI) {
            constexpr int COPIES = BM * RC / 64;
            static_assert((BM * RC) % 64 == 0, "whole copies of the staged tile");
            const int g0 = wave * COPIES / WAVES, g1 = (wave + 1) * COPIES / WAVES;
            const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr);
#pragma unroll
            for (int j = 0; j < (COPIES + WAVES - 1) / WAVES; ++j) {
                const int g = g0 + j;
                if (g < g1) {  // wave-uniform
                    const int q = 64 * g + lane, row = q / RC, c = q - row * RC;
                    const bool ok = c < RC - 1 && m0 + row < a.M && n0 + c * 8 < a.N;
                    lds_copy16(rS, ok ? (uint32_t)(row * a.N + c * 8) * 2 : kOob, 0, base + g * 1024);
                }
            }
        } else {
            static_assert((128 * RC) % 64 == 0, "whole copies of padded rows");
            const int r0 = wm * 128, c0 = wn * WN;
            const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr + (uint32_t)(wave * EPI_WAVE));
#pragma unroll
            for (int j = 0; j < 128 * RC / 64; ++j) {
                const int q = 64 * j + lane, row = q / RC, c = q - row * RC;
                const int col = c0 + c * 8;
                const bool ok = c < RC - 1 && m0 + r0 + row < a.M && n0 + col < a.N;
                lds_copy16(rS, ok ? (uint32_t)((r0 + row) * a.N + col) * 2 : kOob, 0, base + j * 1024);
            }
        }
    }

    // The elements e < cvalid of one 16-byte chunk bound for byte offset
    // off of out (nothing for off == kOob).
    __device__ __forceinline__ static void store_chunk_elems(const u32x4_t v, __amdgpu_buffer_rsrc_t rO, uint32_t off,
                                                             int cvalid) {
        constexpr int EPC = 16 / OES;
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
            if constexpr (OES == 2) {
                const uint16_t h = (uint16_t)((e & 1) ? (v[e >> 1] >> 16) : (v[e >> 1] & 0xffffu));
                store_elem<2>(h, rO, (off != kOob && e < cvalid) ? off + e * 2 : kOob);
            } else {
                const uint8_t b = (uint8_t)(v[e >> 2] >> (8 * (e & 3)));
                __builtin_amdgcn_raw_buffer_store_b8(b, rO, (off != kOob && e < cvalid) ? off + e : kOob, 0, 0);
            }
        }
    }

    __device__ __forceinline__ static void epilogue_lds(const GemmArgs &a, int m0, int n0, int wave, int wm, int wn,
                                                        int lane, const acc_t (&acc)[NRB][NI], FL_LDS char *lds) {
        using io = Io<DT>;
        using quad_t = u32x2_t;
        const size_t o_org = (size_t)m0 * a.N + n0;
        const size_t o_bytes = ((size_t)a.M * a.N - o_org) * 2;  // Y and R, in the I/O dtype
        const __amdgpu_buffer_rsrc_t rO =
            make_rsrc(static_cast<char *>(a.out) + o_org * OES, ((size_t)a.M * a.N - o_org) * OES);
        const __amdgpu_buffer_rsrc_t rY =
            make_rsrc(a.Y ? static_cast<const char *>(a.Y) + o_org * 2 : nullptr, a.Y ? o_bytes : 0);
        // R is the residual, or in the backward epilogue the saved X (same
        // shape, same loads)
        // (a null X -- the plain transposed-B product -- reads as zeros)
        constexpr bool has_r = RES || BWD;
        const void *r_src = BWD ? a.Xs : a.R;
        const bool r_live = has_r && r_src != nullptr;
        const __amdgpu_buffer_rsrc_t rR =
            make_rsrc(r_live ? static_cast<const char *>(r_src) + o_org * 2 : nullptr, r_live ? o_bytes : 0);
        const __amdgpu_buffer_rsrc_t rDY = make_rsrc(
            (BWD && ACT == FL_ACT_GLU) ? static_cast<char *>(a.dY) + o_org * 2 : nullptr,
            (BWD && ACT == FL_ACT_GLU) ? o_bytes : 0);
        const __amdgpu_buffer_rsrc_t rBias =
            make_rsrc(a.bias ? static_cast<const char *>(a.bias) + (size_t)n0 * 2 : nullptr,
                      a.bias ? (size_t)(a.N - n0) * 2 : 0);
        FL_LDS char *wbuf = SHARED_EPI ? lds + (wm * 128) * EPI_ROW + wn * WN * OES : lds + wave * EPI_WAVE;
        const int lrow = lane & (RBH - 1);
        int col[NG], valid[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            col[g] = wn * WN + gcol(g, lane);
            valid[g] = a.N - n0 - col[g];
        }
        float dsum[BWD ? NG : 1][4];  // backward: this lane's column sums of dX
        if constexpr (BWD) {
#pragma unroll
            for (int g = 0; g < NG; ++g)
#pragma unroll
                for (int e = 0; e < 4; ++e) dsum[g][e] = 0.0f;
        }
        quad_t bq[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            bq[g] = quad_t{};
            if (a.bias) bq[g] = base::load4(rBias, valid[g] > 0 ? (uint32_t)col[g] * 2 : kOob, valid[g]);
        }
        auto yoff = [&](int mi, int g) -> uint32_t {
            const int row = wm * 128 + mi * RBH + lrow;
            return (m0 + row < a.M && valid[g] > 0) ? (uint32_t)(row * a.N + col[g]) * 2 : kOob;
        };
        // Y (gate) of row block mi+1 is loaded before row block mi is
        // computed, and so is R (residual) except with the gate, where the
        // registers for two look-ahead rings are not there and R is loaded
        // for the current row block.  Every load precedes the stores of
        // phase 2, so out may alias Y or R.
        constexpr int RA = ACT == FL_ACT_GLU ? 0 : 1;  // residual row blocks loaded ahead
        quad_t yq[2][NG], rq[RA + 1][NG];
        // the side input through LDS (see stage_side)
        const bool slds = SIDE != 0 && (a.N & 7) == 0;
        const bool y_reg = ACT == FL_ACT_GLU && !(SIDE == 1 && slds);
        const bool r_reg = has_r && !((SIDE == 2 || SIDE2) && slds);
        FL_LDS char *wbuf2 = lds + EPI_BYTES + wave * EPI_WAVE;  // SIDE2: the saved X
        if constexpr (SIDE != 0) {
            if (slds) {
                stage_side(a, SIDE == 1 ? a.Y : r_live ? r_src : nullptr, m0, n0, wave, wm, wn, lane,
                           (uint32_t)(uintptr_t)(FL_LDS void *)lds);
                if constexpr (SIDE2)
                    stage_side(a, r_live ? r_src : nullptr, m0, n0, wave, wm, wn, lane,
                               (uint32_t)(uintptr_t)(FL_LDS void *)(lds + EPI_BYTES));
                wait_vm<0>();
                if constexpr (SHARED_EPI) __syncthreads();  // a lane's values were copied by other waves
            }
        }
        if (y_reg) {
#pragma unroll
            for (int g = 0; g < NG; ++g) yq[0][g] = base::load4(rY, yoff(0, g), valid[g]);
        }
        if constexpr (RA && has_r) {
            if (r_reg) {
#pragma unroll
                for (int p = 0; p < RA; ++p)
#pragma unroll
                    for (int g = 0; g < NG; ++g) rq[p][g] = base::load4(rR, yoff(p, g), valid[g]);
            }
        }
#pragma unroll
        for (int mi = 0; mi < NRB; ++mi) {
            if (y_reg && mi + 1 < NRB) {
#pragma unroll
                for (int g = 0; g < NG; ++g) yq[(mi + 1) & 1][g] = base::load4(rY, yoff(mi + 1, g), valid[g]);
            }
            if (r_reg && mi + RA < NRB) {
#pragma unroll
                for (int g = 0; g < NG; ++g)
                    rq[(mi + RA) % (RA + 1)][g] = base::load4(rR, yoff(mi + RA, g), valid[g]);
            }
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const int r = mi * RBH + lrow, c = gcol(g, lane);  // within the wave's tile
                if constexpr (SIDE != 0) {
                    if (slds) {
                        const quad_t s = *(const FL_LDS quad_t *)(wbuf + r * EPI_ROW + c * 2);
                        if constexpr (SIDE == 1)
                            yq[mi & 1][g] = s;
                        else
                            rq[mi % (RA + 1)][g] = s;
                        if constexpr (SIDE2)
                            rq[mi % (RA + 1)][g] = *(const FL_LDS quad_t *)(wbuf2 + r * EPI_ROW + c * 2);
                    }
                }
                float v[4];
                if constexpr (BWD) {
                    // dX = D * act'(X), and for the gate dY = D * X (D: the
                    // accumulator; no bias on this side)
                    float dy[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float y = (ACT == FL_ACT_GLU) ? base::elem_f32(yq[mi & 1][g], e) : 0.0f;
                        const float d = accv(acc, mi, g, e);
                        const float xs = base::elem_f32(rq[mi % (RA + 1)][g], e);
                        float dx = d * activate_grad<ACT>(xs, y);
                        asm("" : "+v"(dx));
                        v[e] = dx;
                        dsum[g][e] += dx;
                        // held in fp32 before the cast, as in activate(): a
                        // multiply folded into a mixed-precision fma with a +0
                        // addend turned -0 (D < 0, X = 0) into +0
                        dy[e] = d * xs;
                        asm("" : "+v"(dy[e]));
                    }
                    if constexpr (ACT == FL_ACT_GLU) {
                        const uint32_t off = yoff(mi, g);
                        u32x2_t w;
                        w[0] = io::pack2(dy[0], dy[1]);
                        w[1] = io::pack2(dy[2], dy[3]);
                        if (valid[g] >= 4) {
                            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u32_t, w), rDY, off, 0, 0);
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                store_elem<2>((uint16_t)(w[e >> 1] >> (16 * (e & 1))), rDY,
                                              (off != kOob && e < valid[g]) ? off + e * 2 : kOob);
                        }
                    }
                } else
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float y = (ACT == FL_ACT_GLU) ? base::elem_f32(yq[mi & 1][g], e) : 0.0f;
                    float x;
                    if constexpr (F8)
                        x = __builtin_fmaf(accv(acc, mi, g, e), a.ab_scale, base::elem_f32(bq[g], e));
                    else
                        x = accv(acc, mi, g, e) + base::elem_f32(bq[g], e);
                    if constexpr (has_r) x += base::elem_f32(rq[mi % (RA + 1)][g], e);
                    v[e] = activate<ACT>(x, y);
                }
                if constexpr (QF < 0) {
                    u32x2_t w;
                    w[0] = io::pack2(v[0], v[1]);
                    w[1] = io::pack2(v[2], v[3]);
                    *(FL_LDS u32x2_t *)(wbuf + r * EPI_ROW + c * 2) = w;
                } else {
                    *(FL_LDS uint32_t *)(wbuf + r * EPI_ROW + c) = quantize4<QF>(v, a.scale);
                }
            }
            // One row block at a time: without this the scheduler reads
            // every accumulator out of the AGPRs up front and spills.
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (SHARED_EPI) {
            __syncthreads();  // every wave's part of the tile is in LDS
        } else {
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's writes are visible to itself
            asm volatile("" ::: "memory");
        }
        // Phase 2, written out here: as a separate (inlined) function it
        // made the register allocator spill in the 256-register kernels.
        // This wave stores P_ROWS rows of P_W output elements, from tile row
        // row0 and column col0, staged at pbase.
        constexpr int P_ROWS = SHARED_EPI ? BM / WAVES : 128;
        constexpr int P_W = SHARED_EPI ? BN : WN;
        constexpr int EPC = 16 / OES;   // output elements per 16-byte chunk
        constexpr int CPR = P_W / EPC;  // 16-byte chunks per staged row
        constexpr int BATCH = 8;        // LDS reads issued ahead of their stores
        const int row0 = SHARED_EPI ? wave * P_ROWS : wm * 128;
        const int col0 = SHARED_EPI ? 0 : wn * WN;
        const FL_LDS char *pbase = SHARED_EPI ? lds + row0 * EPI_ROW : wbuf;
        if constexpr (64 % CPR == 0) {
            constexpr int RPP = 64 / CPR;  // rows per store instruction
            constexpr int PASSES = P_ROWS / RPP;
            static_assert(PASSES % BATCH == 0, "whole batches");
            const int cchunk = lane % CPR;
            const int ccol = col0 + cchunk * EPC;
            const int cvalid = a.N - n0 - ccol;
            const FL_LDS char *rbase = pbase + (lane / CPR) * EPI_ROW + cchunk * 16;
            auto out_off = [&](int rr) -> uint32_t {
                const int row = row0 + rr * RPP + lane / CPR;
                return m0 + row < a.M ? (uint32_t)(row * a.N + ccol) * OES : kOob;
            };
            if (cvalid >= EPC) {
                // Whole 16-byte chunks: BATCH reads, one wait, BATCH stores.
#pragma unroll 1
                for (int rb = 0; rb < PASSES; rb += BATCH) {
                    u32x4_t v[BATCH];
#pragma unroll
                    for (int j = 0; j < BATCH; ++j)
                        v[j] = *(const FL_LDS u32x4_t *)(rbase + (rb + j) * RPP * EPI_ROW);
                    if (a.stream_out) {
#pragma unroll
                        for (int j = 0; j < BATCH; ++j)
                            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32_t, v[j]), rO,
                                                                   out_off(rb + j), 0, kStreamStore);
                    } else {
#pragma unroll
                        for (int j = 0; j < BATCH; ++j)
                            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32_t, v[j]), rO,
                                                                   out_off(rb + j), 0, 0);
                    }
                }
            } else {
                // The chunk that holds column N-1 (and chunks past it): elements.
#pragma unroll 1
                for (int rr = 0; rr < PASSES; ++rr)
                    store_chunk_elems(*(const FL_LDS u32x4_t *)(rbase + rr * RPP * EPI_ROW), rO, out_off(rr), cvalid);
            }
        } else {
            // Rows of CPR chunks, CPR not a divisor of 64: pass p covers
            // chunks 64p .. 64p+63 of this wave's rows in row order, so a
            // store instruction writes 64 / CPR whole rows and pieces of its
            // neighbours' rows, still whole 128-byte lines together.
            constexpr int PASSES = P_ROWS * CPR / 64;
            constexpr int BATCH = PASSES % 8 == 0 ? 8 : PASSES % 6 == 0 ? 6 : 4;
            static_assert(P_ROWS * CPR % 64 == 0 && PASSES % BATCH == 0, "whole passes and batches");
            auto chunk_at = [&](int p, int &row, int &cc) {
                const int q = p * 64 + lane;
                row = q / CPR;
                cc = q % CPR;
            };
            auto out_off = [&](int row, int col) -> uint32_t {
                return m0 + row0 + row < a.M ? (uint32_t)((row0 + row) * a.N + col) * OES : kOob;
            };
            if (a.N - n0 - col0 >= P_W) {
                // every column this wave stores is below N
#pragma unroll 1
                for (int rb = 0; rb < PASSES; rb += BATCH) {
                    u32x4_t v[BATCH];
                    uint32_t off[BATCH];
#pragma unroll
                    for (int j = 0; j < BATCH; ++j) {
                        int row, cc;
                        chunk_at(rb + j, row, cc);
                        v[j] = *(const FL_LDS u32x4_t *)(pbase + row * EPI_ROW + cc * 16);
                        off[j] = out_off(row, col0 + cc * EPC);
                    }
                    if (a.stream_out) {
#pragma unroll
                        for (int j = 0; j < BATCH; ++j)
                            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32_t, v[j]), rO, off[j], 0,
                                                                   kStreamStore);
                    } else {
#pragma unroll
                        for (int j = 0; j < BATCH; ++j)
                            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32_t, v[j]), rO, off[j], 0, 0);
                    }
                }
            } else {
                // the rows reach past column N-1: element stores
#pragma unroll 1
                for (int p = 0; p < PASSES; ++p) {
                    int row, cc;
                    chunk_at(p, row, cc);
                    const int col = col0 + cc * EPC;
                    store_chunk_elems(*(const FL_LDS u32x4_t *)(pbase + row * EPI_ROW + cc * 16), rO,
                                      out_off(row, col), a.N - n0 - col);
                }
            }
        }
        if (BWD && (a.dbias || a.dbias_part)) {
            // Column sums of dX for dbias: the lanes' sums over their 4 rows
            // meet in the wave's LDS area (row lrow, phase 2 has read it
            // already) and lane t adds up column t over the 32 rows.  With a
            // partial-sum buffer that value goes to its row 2*tile_row + wm
            // (a later pass adds the rows in order, so dbias is the same to
            // the bit whatever order the tiles ran in); else one fp32 atomic
            // per column and wave adds it into dbias (the order of those
            // additions across tiles is not fixed).  Rows past M and columns
            // past N contribute zeros (A and B^T read as zero there).
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const int c = gcol(g, lane);
                const f32x4_t t = {dsum[g][0], dsum[g][1], dsum[g][2], dsum[g][3]};
                *(FL_LDS f32x4_t *)(wbuf + lrow * DB_ROW + c * 4) = t;
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
            asm volatile("" ::: "memory");
            float sum = 0.0f;
#pragma unroll 8
            for (int r = 0; r < RBH; ++r) sum += *(const FL_LDS float *)(wbuf + r * DB_ROW + lane * 4);
            const int col = n0 + wn * WN + lane;
            if (col < a.N) {
                if (a.dbias_part)
                    a.dbias_part[(size_t)(2 * (m0 / BM) + wm) * a.N + col] = sum;
                else
                    unsafeAtomicAdd(a.dbias + col, sum);
            }
        }
    }

    __device__ __forceinline__ static void run_tile(const GemmArgs &a, int pid, char *smem) {
        const int tid = threadIdx.x, lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int wm = wave / WAVES_N, wn = wave % WAVES_N;
        int tm, tn;
        grouped_tile(pid, a.tiles_m, a.tiles_n, a.group, tm, tn);
        const int m0 = tm * BM, n0 = tn * BN;
        const FL_LDS char *lds = (const FL_LDS char *)smem;
        const uint32_t lds_addr = (uint32_t)(uintptr_t)(FL_LDS void *)smem;

        acc_t acc[NRB][NI];
#pragma unroll
        for (int mi = 0; mi < NRB; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                for (int e = 0; e < AV; ++e) acc[mi][ni][e] = 0.0f;

        const int nk = (a.K + BK - 1) / BK;
        if (nk > 0) {
            Lane L;
            setup(a, m0, n0, wave, lane, wm, wn, L);
            // Stages 0..NBUF-2 whole, then part 0 of stage NBUF-1's copies
            // (its other parts go out in stage 0's first blocks).
#pragma unroll
            for (int b = 0; b < NBUF - 1; ++b) copy_all(L, stage_of(a, b, wave, lds_addr + b * BUF_BYTES));
            Stage pend = stage_of(a, NBUF - 1, wave, lds_addr + (NBUF - 1) * BUF_BYTES);
            copy_range<0, part_lo(1)>(L, pend);
            wait_vm<(NBUF - 2) * DMA_PER_WAVE + part_lo(1)>();
            if (((a.K | a.N) % EPCH) && nk == 1) fix_k_tail(a, L, m0, n0, 0, wave, lane, (FL_LDS char *)lds);
            __syncthreads();
            Frags f[2];
            read_all(L, lds, 0, f[0]);
            int buf = 0;
            // With SPLIT_TAIL the stages up to nk-3 run without the tail
            // fix-up and the last two from a copy that has it (stage nk-2
            // fixes stage nk-1); otherwise every stage runs the one copy.
            int kt = 0;
            if constexpr (KK % 2 == 0 && !SPLIT_TAIL) {
#pragma unroll 1
                for (; kt < nk; ++kt) {
                    stage<0, 0, true>(a, L, lds, lds_addr, m0, n0, kt, nk, buf, wave, pend, f, acc);
                    buf = buf + 1 == NBUF ? 0 : buf + 1;
                }
            } else if constexpr (KK % 2 == 0) {
#pragma unroll 1
                for (; kt + 2 < nk; ++kt) {
                    stage(a, L, lds, lds_addr, m0, n0, kt, nk, buf, wave, pend, f, acc);
                    buf = buf + 1 == NBUF ? 0 : buf + 1;
                }
                if (kt < nk) {
                    stage<0, 0, true>(a, L, lds, lds_addr, m0, n0, kt, nk, buf, wave, pend, f, acc);
                    buf = buf + 1 == NBUF ? 0 : buf + 1;
                    ++kt;
                }
                if (kt < nk) stage<0, 0, true>(a, L, lds, lds_addr, m0, n0, kt, nk, buf, wave, pend, f, acc);
            } else if constexpr (!SPLIT_TAIL) {
                // an odd number of blocks per stage: two stages per pass, the
                // second starting from the other operand buffer; an odd last
                // stage after the loop (no branch inside the loop body)
#pragma unroll 1
                for (; kt + 1 < nk; kt += 2) {
                    stage<0, 0, true>(a, L, lds, lds_addr, m0, n0, kt, nk, buf, wave, pend, f, acc);
                    buf = buf + 1 == NBUF ? 0 : buf + 1;
                    stage<0, 1, true>(a, L, lds, lds_addr, m0, n0, kt + 1, nk, buf, wave, pend, f, acc);
                    buf = buf + 1 == NBUF ? 0 : buf + 1;
                }
                if (kt < nk) stage<0, 0, true>(a, L, lds, lds_addr, m0, n0, kt, nk, buf, wave, pend, f, acc);
            } else {
                // the same, with the last two or three stages after the loop
#pragma unroll 1
                for (; kt + 3 < nk; kt += 2) {
                    stage<0, 0>(a, L, lds, lds_addr, m0, n0, kt, nk, buf, wave, pend, f, acc);
                    buf = buf + 1 == NBUF ? 0 : buf + 1;
                    stage<0, 1>(a, L, lds, lds_addr, m0, n0, kt + 1, nk, buf, wave, pend, f, acc);
                    buf = buf + 1 == NBUF ? 0 : buf + 1;
                }
                if (kt + 1 < nk) {
                    stage<0, 0, true>(a, L, lds, lds_addr, m0, n0, kt, nk, buf, wave, pend, f, acc);
                    buf = buf + 1 == NBUF ? 0 : buf + 1;
                    stage<0, 1, true>(a, L, lds, lds_addr, m0, n0, kt + 1, nk, buf, wave, pend, f, acc);
                    buf = buf + 1 == NBUF ? 0 : buf + 1;
                    kt += 2;
                }
                if (kt < nk) stage<0, 0, true>(a, L, lds, lds_addr, m0, n0, kt, nk, buf, wave, pend, f, acc);
            }
            // The look-ahead copies (past the end of K) must land before this
            // workgroup's LDS is reused.
            wait_vm<0>();
            __syncthreads();
        }
        // The epilogue's per-lane addresses derive from a copy of the lane
        // index made here, so the compiler cannot compute them before the K
        // loop and keep them (spilled) across it.
        int lane_e = lane;
        asm volatile("" : "+v"(lane_e));
        epilogue_lds(a, m0, n0, wave, wm, wn, lane_e, acc, (FL_LDS char *)smem);
        if (a.tile_count && tid == 0) atomicAdd(&a.tile_count[tm * a.tiles_n + tn], 1u);
    }
};

// Look-ahead copies issued over two blocks: measured best of 1..4 on the
// 4096^3 fp16, 8192x14336x4096 bf16 and 1024x21568x4096 fp16 shapes.
constexpr int kCopySpread = 2;

template <int DT, int ACT, int BK, int BN, int WAVES_N, int SPREAD, int OCC, bool RES, int QF, int IN = DT,
          bool M16 = false>
__global__ void __launch_bounds__(64 * 2 * WAVES_N, OCC) fused_linear_dma16_kernel(GemmArgs a) {
    using T = Dma16<DT, ACT, BK, BN, WAVES_N, SPREAD, OCC, RES, QF, IN, false, M16>;
    __shared__ __attribute__((aligned(1024))) char smem[T::SMEM_BYTES];
    // One strided loop for both launch modes (one program per tile runs one
    // iteration), so the tile body is inlined once.
    const int ntiles = a.tiles_m * a.tiles_n;
    const int G = gridDim.x;
    const int slot = a.xcd_remap ? xcd_logical(blockIdx.x, G) : (int)blockIdx.x;
    for (int pid = slot; pid < ntiles; pid += G) {
        T::run_tile(a, pid, smem);
        __syncthreads();
    }
}

// The backward epilogue kernel ("Optimizing GEMM + Activation on CDNA4 with
// TLX", "Future Work": the epilogue fusion in the backward pass): D = A @
// B^T with B given as (N, K) row-major, then dX = D * act'(Xs), the gate's
// dY = D * Xs, and dbias += column sums of dX.  Same tile body and launch
// loop as the forward kernel.
template <int DT, int ACT, int BK, int BN, int WAVES_N, bool M16 = false>
__global__ void __launch_bounds__(64 * 2 * WAVES_N, 1) fused_linear_bwd_kernel(GemmArgs a) {
    using T = Dma16<DT, ACT, BK, BN, WAVES_N, kCopySpread, 1, false, -1, DT, true, M16>;
    __shared__ __attribute__((aligned(1024))) char smem[T::SMEM_BYTES];
    const int ntiles = a.tiles_m * a.tiles_n;
    const int G = gridDim.x;
    const int slot = a.xcd_remap ? xcd_logical(blockIdx.x, G) : (int)blockIdx.x;
    for (int pid = slot; pid < ntiles; pid += G) {
        T::run_tile(a, pid, smem);
        __syncthreads();
    }
}

}  // namespace fl
