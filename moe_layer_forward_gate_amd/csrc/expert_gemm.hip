// Expert compute on bf16 MFMA: grouped GEMMs over the by-expert row order.
//
// [hotelren §2.1 steps 4-5] each chosen expert's weights are loaded and its
// matrix products run; [0539edu §2.2] expert weights are stored expert-major and
// consecutively, and the kernel keeps weight slices in on-chip memory;
// [hotelren §2.3] expert_gemm_kernel is tailored to the expert weight layout;
// [mhpq §3.3] tensor-core fragments in 16x16 tiles on the original hardware.
//
// Up:   H[p, f] = silu(x[t(p)] . Wg[e][:, f]) * (x[t(p)] . Wu[e][:, f])
// Down: O[c(p), n] = wgt(c) * (H[p] . Wd[e][:, n]); wgt is the routing weight of
//       slot c (or the shared gate for a shared slice), so the top-k weighting of
//       the Gather stage is applied in this epilogue ([pptc §2.1] fused
//       aggregation).
//
// Workgroup tile BM x 256 (BM = 256 on 16 waves for bf16 weights, 128 on 8 waves
// for int8, 64 on 8 waves for int4); each wave owns a 64 x 64 block of
// v_mfma_f32_16x16x32_bf16 accumulators (int4: 32 x 64). K step 32 (bf16 weights), 64
// (int8) or 128 (int4), four LDS stages, three K steps of loads in flight, one barrier
// per step. Operands are
// staged in LDS in MFMA fragment order: one 1 KB block = 16 rows x 32 K, lane l
// holding row l%16, K 8*(l/16)..+7, so every fragment read is a conflict-free
// 16-byte-per-lane ds_read. Global -> LDS traffic uses the gfx950 LDS-DMA load
// (global_load_lds_dwordx4): each wave instruction fills one whole 1 KB block,
// lane l fetching its own 16 bytes. Both operands are stored in that fragment
// order in HBM, so every block is one contiguous 1 KB read (sixteen separate
// 64-byte row pieces per block, as a gather from token rows would need, keep the
// vector memory pipe busy for about twice as long per byte): the A operand of the
// up projection is packed by launch_pack_a after the scatter, the up kernel's
// epilogue writes H in the down projection's A order, and expert weights are
// packed at create time (bf16: [Et][N/16][K/32][64][8]).
// int8 weights ([E][N/16][K/64][64][16], bytes 0-7 the first 32-K half) are staged
// in LDS as int8 by the same LDS-DMA (half the bytes of bf16) and widened to bf16 in
// registers right before their MFMAs (exact: |q| <= 127 fits bf16's significand);
// their per-column scale multiplies the fp32 accumulator in the epilogue.
// int4 weights ([E][N/16][K/128][64][16 B], one 1 KB block per 16 columns and 128-row
// scale group) take one K step per group: a stage holds the group's A blocks, the int4
// blocks and the group's 256 column scales (one more 1 KB block, its eighths loaded by
// the eight waves). Each code u = q + 8 is placed in the low mantissa bits of bf16 128.0
// (one mask-and-or per pair of values), so the MFMAs form sum(a * (q + 136)); one more
// MFMA of the token fragments against the constant 136 gives 136 * sum(a), and the
// group's partial, less that, times the column's group scale is added in fp32.
// Up-projection columns are packed gate/up interleaved per 16 columns, so each
// lane holds the gate and up accumulators of the same (row, f) and SiLU * up
// runs in registers.
#include <type_traits>

#include "common.h"

namespace moe {
namespace {

constexpr int BN = 256;
constexpr int kBf16Waves = 16;
constexpr int GN = 4;       // column tiles per group (see decode_tile), or all of them when at most kGNAll

// Column tiles per group: 4, or every column tile of the projection when there are at most
// 6 (one group spans the expert's width, so each row tile's A operand is read by all its
// column tiles together: the skewed 128-expert layer's up projection, 6 column tiles,
// 235 -> 200 us; its down projection, 8 column tiles, ran 167 us in groups of 4 against
// 171 in one group of 8).
constexpr int kGNAll = 6;
// Tiles dealt to the XCDs in chunks of 32 (decode_tile_at): against one contiguous stretch
// per XCD, 8-expert layer T = 4096 2.76 -> 2.68 ms, int8 T = 256 0.69 -> 0.67 ms, int4
// T = 256 0.79 -> 0.75 ms, the shared + fine and skewed layers within 1%; chunks of 64
// were slower than one stretch, chunks of 16 about as fast as 32.
constexpr int kXcdChunk = 32;
__host__ __device__ __forceinline__ int col_group(int nt) { return nt <= kGNAll ? nt : GN; }

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint32_t i8x2_to_bf16x2(uint32_t w, int sh) {
    // bytes sh/8 and sh/8+1 of w as two bf16 (exact widening of small integers)
    const float f0 = (float)(int)(int8_t)(w >> sh);
    const float f1 = (float)(int)(int8_t)(w >> (sh + 8));
    // the high halves of the two fp32 patterns (exact: |q| <= 128 has at most 8 significant
    // bits), picked by one byte permute: bytes 2-3 of f0, then bytes 2-3 of f1
    return __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
}

__device__ __forceinline__ u32x4 i8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
    return u32x4{i8x2_to_bf16x2(lo, 0), i8x2_to_bf16x2(lo, 16), i8x2_to_bf16x2(hi, 0), i8x2_to_bf16x2(hi, 16)};
}

// one 16-byte LDS-DMA load per lane: LDS[block + 16*lane] = *src (block is wave-uniform)
__device__ __forceinline__ void dma16(const void* src, u32x4* lds_block) {
    __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_block, 16, 0, 0);
}
// the same with the non-temporal cache policy: weight blocks no other row tile will read
__device__ __forceinline__ void dma16_nt(const void* src, u32x4* lds_block) {
    __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_block, 16, 0, 2);
}

// s_waitcnt with vmcnt <= N (N < 64) and the other counters left alone (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ __forceinline__ void wait_vm_le() {
    static_assert(N >= 0 && N < 64, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier without a memory fence (the waits above it are explicit); the
// memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Pipeline shape: both operands stream through LDS-DMA, four stages (three K steps of
// loads in flight). bf16: K step 32. int8: K step 64 (one 1 KB int8 block holds 16
// columns x 64 K), widened to bf16 when the wave reads its B fragments from LDS.
// int4: K step 128 (one scale group).
template <int WQ> struct Pipe;
template <> struct Pipe<kWBf16> { static constexpr int BK = 32, STAGES = 4; };
template <> struct Pipe<kWI8> { static constexpr int BK = 64, STAGES = 4; };
template <> struct Pipe<kWI4> { static constexpr int BK = 128, STAGES = 4; };

// Wave layout: NW waves with 64-row wave tiles: 16 waves tile a 256-row block 4 x 4
// (64 x 64 wave tiles, four waves per SIMD, 128 registers each); 8 waves tile a 128-row
// block 2 x 4 (64 x 64) or a 256-row block 4 x 2 (64 x 128); 4 waves would tile it 2 x 2
// with (BM/2)-row x 128-column wave tiles; 8 waves tile a 64-row block 2 x 4 (32 x 64).
template <int BM, int NW>
struct WaveShape {
    static constexpr int WM = NW >= 8 ? (BM >= 128 ? BM / 64 : 2) : 2;  // waves along M
    static constexpr int WN = NW / WM;                // waves along N
    static constexpr int MWB = BM / 16 / WM;          // 16-row blocks per wave
    static constexpr int NBW = (BN / 16) / WN;        // 16-column blocks per wave
};

template <int BM, int NW, int WQ, bool UP>
__global__ __launch_bounds__(NW * 64, 1) void expert_gemm(GemmArgs a) {
    constexpr bool INT8 = WQ == kWI8;
    constexpr bool INT4 = WQ == kWI4;
    constexpr int kThreads = NW * 64;
    constexpr int kWaves = NW;
    constexpr int BK = Pipe<WQ>::BK;
    constexpr int STAGES = Pipe<WQ>::STAGES;
    constexpr int KH = BK / 32;               // 32-K halves per K step
    constexpr int MBLK = BM / 16;             // 16-row blocks per tile
    constexpr int WM = WaveShape<BM, NW>::WM;
    constexpr int WN = WaveShape<BM, NW>::WN;
    constexpr int MWB = WaveShape<BM, NW>::MWB;
    constexpr int NBW = WaveShape<BM, NW>::NBW;
    constexpr int ABLK = MBLK * KH;           // A blocks per stage
    constexpr int BBLK = INT8 || INT4 ? BN / 16 : (BN / 16) * KH;  // B blocks per stage (int8/int4: one spans BK)
    constexpr int SBLK = INT4 ? 1 : 0;        // int4: the group's column scales
    constexpr int STAGE = ABLK + BBLK + SBLK; // 1 KB blocks per stage
    static_assert(!INT4 || kWaves == 8, "int4 scales: one eighth of the block per wave");
    constexpr int AW = ABLK / kWaves;         // A block loads per wave per stage
    constexpr int BW = BBLK / kWaves;         // B block loads per wave per stage
    constexpr int LPS = AW + BW + SBLK;       // LDS-DMA loads per wave per stage

    const int K = UP ? a.d : a.F;
    const int N = UP ? 2 * a.F : a.d;
    // column tiles; the last one is partial when N % 256 == 128 (N is a multiple of 128):
    // its missing 16-column blocks load the expert's last block and are never stored, and
    // since they come in whole wave shares (multiples of 8 blocks), a wave is either all
    // valid or all skipped
    const int NT = (N + BN - 1) / BN;
    const int NB16 = N / 16;  // valid 16-column blocks
    const int S = UP ? 1 : a.ksplit;
    Tile tl;
    int split = 0;
    int kv = 1;  // shared slices this tile sums as one K (merged shared down projection)
    if (!UP && a.merge_shared) {
        if (!decode_tile_down_merged(a.tile_start, a.offsets, a.Et - (a.kt - a.k), a.kt - a.k, NT, col_group(NT), BM,
                                     tl, kv))
            return;
    } else {
        // split-K: logical tile index = tile * S + split
        if (!decode_tile_split(a.tile_start, a.offsets, a.Et, NT, col_group(NT), BM, S, tl, split, kXcdChunk))
            return;
    }
    const int Kpart = K / S;
    const int kbase = split * Kpart;

    extern __shared__ u32x4 lds[];  // [STAGES][STAGE blocks][64 lanes]

    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int wm = wave / WN, wn = wave % WN;

    // ---- A: wave loads stage blocks b = wave + 8*i: m-block b / KH, K half b % KH. The
    // operand is in fragment order over padded rows (tile g owns row blocks g*BM/16 ..),
    // so every block is one contiguous 1 KB; rows past the expert's last row are zeros.
    // Shared virtual experts past the first read the first one's token rows (the same
    // tokens in the same order).
    const int KA = K / 32;  // 32-K blocks per row block
    const int e0 = a.Et - a.kt + a.k;  // first shared virtual expert (== Et without one)
    const int ga = (UP && tl.e > e0) ? tl.g - a.tile_start[tl.e] + a.tile_start[e0] : tl.g;
    const bf16_t* a_blk[AW];
#pragma unroll
    for (int i = 0; i < AW; ++i) {
        const int b = wave + kWaves * i;
        const size_t mbg = (size_t)ga * (BM / 16) + b / KH;
        a_blk[i] = (UP ? a.xp : a.h) + ((mbg * KA + kbase / 32 + b % KH) * 64 + lane) * 8;
    }
    // ---- B
    const int KS = K / 32;
    const u32x4* b_src;
    const u32x4* s_src = nullptr;  // int4: this lane's 16 bytes of the first group's column scales
    if constexpr (INT8 || INT4) {
        const uint8_t* wb = (const uint8_t*)(UP ? a.wgu : a.wdn) + (size_t)tl.e * N * K / (INT4 ? 2 : 1);
        b_src = reinterpret_cast<const u32x4*>(wb) + kbase / BK * 64;
        if constexpr (INT4) {
            // scales [E][K/128][N] (up: packed column order); a partial last column tile
            // holds N % 256 = 128 columns, read by lanes 0-31 (the other lanes repeat lane 31)
            const int ls = min(lane, (min(BN, N - tl.n * BN) / 4) - 1);
            s_src = reinterpret_cast<const u32x4*>((UP ? a.s_gate : a.s_down) +
                                                   ((size_t)tl.e * (K / BK) + kbase / BK) * N + (size_t)tl.n * BN) + ls;
        }
    } else {
        const bf16_t* wb = (const bf16_t*)(UP ? a.wgu : a.wdn) + (size_t)tl.e * N * K;
        b_src = reinterpret_cast<const u32x4*>(wb) + kbase / 32 * 64;
    }
    // A merged tile runs kv * KBv K steps: step kt is step kt % KBv of slice kt / KBv, whose
    // A rows (the same tokens) and weights lie a fixed stride further on (slices are
    // consecutive virtual experts with equal row-tile counts). kt / KBv by a multiply with
    // ceil(2^32 / KBv), exact for kt * KBv < 2^32.
    const uint32_t KBv = Kpart / BK;
    const uint64_t kb_magic = ((1ull << 32) + KBv - 1) / KBv;
    size_t strideA = 0, strideB = 0;
    if (!UP && kv > 1) {
        strideA = (size_t)(a.tile_start[tl.e + 1] - a.tile_start[tl.e]) * (BM / 16) * KA * 512;
        strideB = (size_t)N * K / 8;  // one expert's weights in 16-byte units (bf16)
    }
    // NA: how many of this wave's A block loads are made. Load i fills row block
    // (wave + NW*i) / KH, read only by the waves of row group (that block) / MWB; a block
    // whose readers hold no rows (past the expert's last row) is not loaded. Blocks grow
    // with i, so the loads made are always a prefix.
    auto issue = [&](int kt, int stage, auto na, auto nt) __attribute__((always_inline)) {
        constexpr int NA = decltype(na)::value;
        constexpr bool NTB = decltype(nt)::value;
        u32x4* st = lds + (size_t)stage * STAGE * 64;
        size_t oa = 0, ob = 0;
        if constexpr (!UP) {
            const uint32_t v = (uint32_t)(((uint64_t)(uint32_t)kt * kb_magic) >> 32);
            kt -= (int)(v * KBv);
            oa = v * strideA;
            ob = v * strideB;
        }
#pragma unroll
        for (int i = 0; i < NA; ++i) dma16(a_blk[i] + oa + (size_t)kt * KH * 512, st + (wave + kWaves * i) * 64);
#pragma unroll
        for (int j = 0; j < BW; ++j) {
            const int blk = wave * BW + j;  // bf16: n-block blk / KH, K half blk % KH; int8: n-block blk
            if constexpr (INT8 || INT4) {
                const int nbg = min(tl.n * (BN / 16) + blk, NB16 - 1);
                const u32x4* src = b_src + ob + ((size_t)nbg * (K / BK) + kt) * 64 + lane;
                if constexpr (NTB) dma16_nt(src, st + (ABLK + blk) * 64);
                else dma16(src, st + (ABLK + blk) * 64);
            } else {
                const int nb = blk / KH, kh = blk % KH;
                const int nbg = min(tl.n * (BN / 16) + nb, NB16 - 1);
                dma16(b_src + ob + ((size_t)nbg * KS + kt * KH + kh) * 64 + lane, st + (ABLK + blk) * 64);
            }
        }
        // int4: the group's 256 column scales, lanes 8w..8w+7 of wave w (every wave makes
        // one load instruction per stage, so the vmcnt bookkeeping is the same for all)
        if constexpr (INT4) {
            if ((lane >> 3) == wave) dma16(s_src + (size_t)kt * (N / 4), st + (ABLK + BBLK) * 64);
        }
    };

    f32x4 acc[MWB][NBW];
#pragma unroll
    for (int i = 0; i < MWB; ++i)
#pragma unroll
        for (int j = 0; j < NBW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int KT = kv * (Kpart / BK);
    {
        // Fragments are double-buffered in registers: the LDS reads of K step kt+1 are
        // issued before the MFMAs of step kt, so LDS latency hides under the MFMAs.
        // Stage (kt-1) % STAGES is refilled in iteration kt: its fragments were read
        // in iteration kt-2 and consumed in kt-1, before this iteration's barrier.
        // B fragments are kept as loaded (int8 bytes are widened right before their MFMAs).
        static_assert(STAGES >= 3, "pipeline shape");
        using BFrag = std::conditional_t<INT8, u32x4, bf16x8>;  // int8 bytes are widened at use
        bf16x8 fa[2][MWB][KH];
        BFrag fb[2][NBW];
        // MA: row blocks of the wave that hold rows (a prefix); the others are neither read
        // nor multiplied
        auto read_frags = [&](int stage, bf16x8 (&af)[MWB][KH], BFrag (&bq)[NBW], auto ma) {
            constexpr int MA = decltype(ma)::value;
            const u32x4* la = lds + (size_t)stage * STAGE * 64;
            const u32x4* lb = la + ABLK * 64;
#pragma unroll
            for (int mb = 0; mb < MA; ++mb)
#pragma unroll
                for (int kh = 0; kh < KH; ++kh)
                    af[mb][kh] = __builtin_bit_cast(bf16x8, la[((wm * MWB + mb) * KH + kh) * 64 + lane]);
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) bq[nb] = __builtin_bit_cast(BFrag, lb[(wn * NBW + nb) * 64 + lane]);
        };
        auto mfma_frags = [&](const bf16x8 (&af)[MWB][KH], const BFrag (&bq)[NBW], auto ma) {
            constexpr int MA = decltype(ma)::value;
            if constexpr (INT8) {
                // column block outermost: each widened B fragment serves every row block
#pragma unroll
                for (int kh = 0; kh < KH; ++kh)
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb) {
                        // int8 lane bytes 0-7: K half 0, bytes 8-15: K half 1
                        const bf16x8 bw = __builtin_bit_cast(bf16x8, kh ? i8x8_to_bf16x8(bq[nb].z, bq[nb].w)
                                                                        : i8x8_to_bf16x8(bq[nb].x, bq[nb].y));
#pragma unroll
                        for (int mb = 0; mb < MA; ++mb)
                            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mb][kh], bw, acc[mb][nb], 0, 0, 0);
                    }
            } else {
#pragma unroll
                for (int mb = 0; mb < MA; ++mb)
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb)
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mb][0], bq[nb], acc[mb][nb], 0, 0, 0);
            }
        };
        // int4: one K step is one scale group; its fragments are read from the stage as they
        // are needed (stage k is complete from iteration k-1's barrier on and is refilled
        // only after iteration k+1's barrier).
        uint32_t nib_mask = 0x000F000Fu;  // held in a register: one v_and_or_b32 per pair
        if constexpr (INT4) asm volatile("" : "+v"(nib_mask));
        auto mfma_i4 = [&](int stage, auto ma) __attribute__((always_inline)) {
            constexpr int MA = decltype(ma)::value;
            const u32x4* la = lds + (size_t)stage * STAGE * 64;
            const u32x4* lb = la + ABLK * 64;
            const float* ls = reinterpret_cast<const float*>(lb + BBLK * 64);
            const bf16x8 k136 = __builtin_bit_cast(bf16x8, u32x4{0x43084308u, 0x43084308u, 0x43084308u, 0x43084308u});
            u32x4 bq[NBW];
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) bq[nb] = lb[(wn * NBW + nb) * 64 + lane];
            f32x4 g[MA][NBW], zr[MA];
#pragma unroll
            for (int kh = 0; kh < KH; ++kh) {
                bf16x8 af[MA];
#pragma unroll
                for (int mb = 0; mb < MA; ++mb)
                    af[mb] = __builtin_bit_cast(bf16x8, la[((wm * MWB + mb) * KH + kh) * 64 + lane]);
#pragma unroll
                for (int mb = 0; mb < MA; ++mb)
                    zr[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mb], k136, kh ? zr[mb] : f32x4{0.f, 0.f, 0.f, 0.f},
                                                                     0, 0, 0);
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) {
                    // word kh of the lane's chunk: K rows 32 kh + 8 (lane / 16) + 0..7 of its column
                    const uint32_t w = bq[nb][kh];
                    const bf16x8 bw = __builtin_bit_cast(
                        bf16x8, u32x4{(w & nib_mask) | 0x43004300u, ((w >> 4) & nib_mask) | 0x43004300u,
                                      ((w >> 8) & nib_mask) | 0x43004300u, ((w >> 12) & nib_mask) | 0x43004300u});
#pragma unroll
                    for (int mb = 0; mb < MA; ++mb)
                        g[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            af[mb], bw, kh ? g[mb][nb] : f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                }
            }
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const float sc = ls[(wn * NBW + nb) * 16 + lane % 16];
#pragma unroll
                for (int mb = 0; mb < MA; ++mb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[mb][nb][i] = fmaf(sc, g[mb][nb][i] - zr[mb][i], acc[mb][nb][i]);
            }
        };
        // Branch-free steady state (a join in the loop would make the compiler drain every
        // LDS read before the MFMAs): every step issues one stage of LDS-DMA loads -- past
        // the last stage it re-loads the last stage into the free slot, which is never
        // read -- and reads the next step's fragments. Steps run in pairs so the register
        // buffer parity is static; one or two steps remain after the pairs.
        // In the ragged last row tile of an expert a wave reads and multiplies only its
        // row blocks that hold rows (MA of MWB; none when all its rows lie past the
        // expert's last row): it still loads its share of the tiles and meets every barrier.
        auto run = [&](auto ma, auto nac, auto nt) __attribute__((always_inline)) {
            constexpr bool C = decltype(ma)::value > 0;
            constexpr int L = decltype(nac)::value + BW + SBLK;  // LDS-DMA loads per stage of this wave
            auto step = [&](int k, auto& ca, auto& cb, auto& na, auto& nb) __attribute__((always_inline)) {
                wait_vm_le<(STAGES - 3) * L>();    // stage k+1 has landed
                lds_barrier();                     // ... for every wave; stage k-1 is free
                issue(min(k + STAGES - 1, KT - 1), (k + STAGES - 1) % STAGES, nac, nt);
                if constexpr (C && INT4) {
                    mfma_i4(k % STAGES, ma);
                } else if constexpr (C) {
                    read_frags((k + 1) % STAGES, na, nb, ma);
                    mfma_frags(ca, cb, ma);
                }
            };
#pragma unroll
            for (int s0 = 0; s0 < STAGES - 1; ++s0) issue(min(s0, KT - 1), s0, nac, nt);
            wait_vm_le<(STAGES - 2) * L>();
            lds_barrier();
            if constexpr (C && !INT4) read_frags(0, fa[0], fb[0], ma);
            int k = 0;
            for (; k + 2 < KT; k += 2) {
                step(k, fa[0], fb[0], fa[1], fb[1]);
                step(k + 1, fa[1], fb[1], fa[0], fb[0]);
            }
            // one or two steps left (bf16: always two, K/32 is even): the last pair step runs
            // in either case (with one step left its fragment read is of a stage that does
            // not exist and is dropped)
            step(k, fa[0], fb[0], fa[1], fb[1]);
            if constexpr (C && INT4) {
                if (KT - k == 2) mfma_i4((k + 1) % STAGES, ma);  // stage k+1 landed before step k's barrier
            } else if constexpr (C) {
                if (!INT8 || KT - k == 2) mfma_frags(fa[1], fb[1], ma);
            }
        };
        const bool has_rows = wm * MWB * 16 < tl.rows;
        int nA = 0;
#pragma unroll
        for (int i = 0; i < AW; ++i)
            if (((wave + kWaves * i) / KH / MWB) * MWB * 16 < tl.rows) nA = i + 1;
        static_assert(AW >= 1 && AW <= 2, "A loads per wave");
        static_assert(MWB >= 2, "row blocks per wave");
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, AW>;  // == 2 when AW == 2
        using MF = std::integral_constant<int, MWB>;
        using NT0 = std::false_type;
        if constexpr (INT8 || INT4) {
            // row blocks holding rows: 0, 1, 2 or all (3 rounds up to all; int4 waves hold two).
            // An expert with one row tile is the only reader of its weights: they are loaded
            // with the non-temporal policy (int8 T = 64 / 128 / 256 layers 478 / 532 / 653 ->
            // 458 / 521 / 635 us); weights several row tiles read stay cached (the same policy
            // for all of them made T = 1024 5% slower).
            const int rw = tl.rows - wm * MWB * 16;
            const bool once = a.tile_start[tl.e + 1] - a.tile_start[tl.e] == 1;
            auto run_nac = [&](auto ma) __attribute__((always_inline)) {
                auto go = [&](auto nt) __attribute__((always_inline)) {
                    if (nA == AW) run(ma, I2{}, nt);
                    else if (nA == 1) run(ma, I1{}, nt);
                    else run(ma, I0{}, nt);
                };
                if (once) go(std::true_type{});
                else go(NT0{});
            };
            if constexpr (MWB == 2) {
                if (rw > 16) run_nac(MF{});
                else if (rw > 0) run_nac(std::integral_constant<int, 1>{});
                else run_nac(I0{});
            } else {
                if (rw > 32) run_nac(MF{});
                else if (rw > 16) run_nac(std::integral_constant<int, 2>{});
                else if (rw > 0) run_nac(std::integral_constant<int, 1>{});
                else run_nac(I0{});
            }
        } else if (has_rows) {
            // bf16 tiles are MFMA-bound and full but for each expert's last one, which is
            // bound by its weight loads: all or none of a wave's row blocks
            if (nA == AW) run(MF{}, I2{}, NT0{});
            else if (nA == 1) run(MF{}, I1{}, NT0{});
            else run(MF{}, I0{}, NT0{});
        } else {
            if (nA == AW) run(I0{}, I2{}, NT0{});
            else if (nA == 1) run(I0{}, I1{}, NT0{});
            else run(I0{}, I0{}, NT0{});
        }
        wait_vm_le<0>();  // no LDS-DMA write may outlive the workgroup
    }

    // ---- epilogue. Lane holds column lane%16 of each 16x16 block, rows 4*(lane/16)+i;
    // results go through a per-wave LDS patch so that global stores are 16 bytes per lane
    // along output rows.
    const int col16 = lane % 16;
    const int rq = 4 * (lane / 16);
    const int rw0 = wm * MWB * 16;  // first tile row of this wave
    __syncthreads();                // every wave is done with the operand stages
    if (tl.n * (BN / 16) + wn * NBW >= NB16) return;  // columns past N (partial last tile): nothing to store
    if constexpr (UP) {
        // H patch: 16*MWB rows x 8*NBW bf16 columns (the wave's NBW/2 gate/up pairs)
        constexpr int PW = 8 * NBW;
        bf16_t* patch = reinterpret_cast<bf16_t*>(lds) + (size_t)wave * (16 * MWB) * PW;
#pragma unroll
        for (int q = 0; q < NBW / 2; ++q) {
            float sg = 1.f, su = 1.f;
            if constexpr (INT8) {
                const int f = ((tl.n * (BN / 16) + wn * NBW) / 2 + q) * 16 + col16;
                sg = a.s_gate[(size_t)tl.e * a.F + f];
                su = a.s_up[(size_t)tl.e * a.F + f];
            }
#pragma unroll
            for (int mb = 0; mb < MWB; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float g = acc[mb][2 * q][i] * sg;
                    const float u = acc[mb][2 * q + 1][i] * su;
                    patch[(mb * 16 + rq + i) * PW + q * 16 + col16] = f32_to_bf16(silu(g) * u);
                }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the patch is written
        // H in the down kernel's fragment order: block (row block, 32-column block), lane l
        // holding row l%16, columns 8*(l/16)..+7. Every row of the tile is written (rows past
        // the expert's last row come out zero from their zero inputs), so the down kernel
        // never reads memory this forward did not write.
        const int fb0 = ((tl.n * (BN / 16) + wn * NBW) / 2) * 16 / 32;
        constexpr int FB = PW / 32;  // 32-column blocks per patch
        static_assert(PW % 32 == 0, "patch width");
#pragma unroll
        for (int mb = 0; mb < MWB; ++mb)
#pragma unroll
            for (int fb = 0; fb < FB; ++fb) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(patch + (mb * 16 + lane % 16) * PW + fb * 32 +
                                                                8 * (lane / 16));
                const size_t blk = ((size_t)tl.g * (BM / 16) + wm * MWB + mb) * (a.F / 32) + fb0 + fb;
                *reinterpret_cast<u32x4*>(a.h + (blk * 64 + lane) * 8) = v;
            }
    } else {
        // output patch: 16*MWB rows x 32 fp32 columns, two 16-column blocks at a time
        float* patch = reinterpret_cast<float*>(lds) + (size_t)wave * (16 * MWB) * 32;
#pragma unroll
        for (int nh = 0; nh < NBW / 2; ++nh) {
#pragma unroll
            for (int mb = 0; mb < MWB; ++mb)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) patch[(mb * 16 + rq + i) * 32 + j * 16 + col16] = acc[mb][2 * nh + j][i];
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
            const int n0 = tl.n * BN + (wn * NBW + 2 * nh) * 16;
#pragma unroll
            for (int c = lane; c < 16 * MWB * 8; c += kWave) {
                const int r = c / 8, c4 = (c % 8) * 4;
                if (rw0 + r < tl.rows) {
                    const int cs = a.sorted_c[tl.seg0 + tl.row0 + rw0 + r];
                    const int t = cs / a.kt, j = cs - t * a.kt;
                    const float wgt = j < a.k ? a.topk_w[(size_t)t * a.k + j] : a.gs[t];
                    f32x4 v = *reinterpret_cast<const f32x4*>(patch + r * 32 + c4) * wgt;
                    if constexpr (INT8) v *= *reinterpret_cast<const f32x4*>(a.s_down + (size_t)tl.e * a.d + n0 + c4);
                    // partial sum `split` of slot cs: row cs*S + split of the combine buffer
                    *reinterpret_cast<f32x4*>(a.ow + ((size_t)cs * S + split) * a.d + n0 + c4) = v;
                }
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // patch reads done before the next half overwrites it
        }
    }
}

template <int BM, int NW, int WQ, bool UP>
hipError_t launch(const GemmArgs& a, hipStream_t s) {
    constexpr int BK = Pipe<WQ>::BK;
    constexpr int KH = BK / 32;
    constexpr int STAGE = (BM / 16) * KH + (WQ != kWBf16 ? BN / 16 : (BN / 16) * KH) + (WQ == kWI4 ? 1 : 0);  // as in the kernel
    static_assert(Pipe<WQ>::STAGES * STAGE * 1024 <= 160 * 1024, "LDS");
    const size_t lds_bytes = (size_t)Pipe<WQ>::STAGES * STAGE * 64 * 16;
    auto kern = expert_gemm<BM, NW, WQ, UP>;
    static bool attr_set = false;  // one-time opt-in above the default dynamic LDS limit
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)lds_bytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int N = UP ? 2 * a.F : a.d;
    const int S = UP ? 1 : a.ksplit;
    const int Kpart = (UP ? a.d : a.F) / S;
    // whole K steps (an even count of 32-K steps for bf16)
    if (Kpart % std::max(BK, 64) != 0 || Kpart < std::max(BK, 64)) return hipErrorInvalidValue;
    if (WQ == kWI4 && (N % 128 != 0 || a.merge_shared)) return hipErrorInvalidValue;
    const int gn = col_group((N + BN - 1) / BN);
    const int NTp = ((N + BN - 1) / BN + gn - 1) / gn * gn;
    // a multiple of 8 workgroups, so every XCD gets ceil(tiles / 8) slots (a merged shared
    // down projection starts its routed tiles at the next multiple of 8 after its own)
    // (+ kXcds * kXcdChunk: the chunked deal needs the tile count rounded up to whole chunks)
    const size_t blocks =
        (size_t)a.max_tiles * NTp * S + (!UP && a.merge_shared ? 2 * kXcds : 0) + kXcds * kXcdChunk;
    dim3 grid((unsigned)((blocks + kXcds - 1) / kXcds * kXcds));
    hipLaunchKernelGGL(kern, grid, dim3(NW * 64), lds_bytes, s, a);
    return hipGetLastError();
}

template <bool UP>
hipError_t launch_dispatch(const GemmArgs& a, int wq, hipStream_t s) {
    // bf16 weights: 256-row tiles on 16 waves (four per SIMD hide more latency than two
    // waves with 64 x 128 tiles, though they read a third more LDS per MFMA); int8: 128-row
    // tiles on 8 waves (two K halves of int8 fragments need the registers of two waves per
    // SIMD). Measured slower: 4 waves with 128 x 128 wave tiles (one wave per SIMD hides
    // nothing), 128-row bf16 tiles (more operand traffic per MFMA). int4, and int8 batches
    // of at most ~24 rows per expert: 64-row tiles on 8 waves (32 x 64 wave tiles).
    if (wq == kWBf16 && a.bm == 256) return launch<256, kBf16Waves, kWBf16, UP>(a, s);
    if (wq == kWI8 && a.bm == 128) return launch<128, 8, kWI8, UP>(a, s);
    if (wq == kWI8 && a.bm == 64) return launch<64, 8, kWI8, UP>(a, s);
    if (wq == kWI4 && a.bm == 64) return launch<64, 8, kWI4, UP>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_expert_up_tiled(const GemmArgs& a, int wq, hipStream_t s) {
    return launch_dispatch<true>(a, wq, s);
}

hipError_t launch_expert_down_tiled(const GemmArgs& a, int wq, hipStream_t s) {
    return launch_dispatch<false>(a, wq, s);
}

}  // namespace moe
