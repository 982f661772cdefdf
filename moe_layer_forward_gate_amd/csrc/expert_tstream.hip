// Expert compute for mid-size batches: row tiles in LDS, weights streamed into registers.
//
// Between decode and prefill an expert holds tens to a few hundred rows and its weights
// are still most of the traffic ([hotelren §2.1]: the bottleneck is moving data). Here
// each wave owns four 16-column weight blocks (two in the int8 down projection while the
// experts average at most 64 rows) and streams them from HBM over the whole K range as
// contiguous 1 KB chunks straight into MFMA operand registers (no LDS round trip; a
// quantised weight byte is widened once), while the workgroup's row tile (up to 128 rows)
// is staged in LDS by LDS-DMA, K step by K step, and read by all four waves: every wave
// multiplies every row of the tile against its own columns.
//   - Workgroup = (row tile, 256 or 128 columns, K split), 4 waves; the tile list, the
//     padded A operand (xp for the up projection, packed H for the down projection) and
//     the outputs are those of the LDS-tiled kernels, so the two are interchangeable.
//   - R K steps of loads are in flight per wave (2 to 4, the most the registers hold beside
//     the tile's accumulators; weights into a ring of R register sets, row blocks into R + 1
//     LDS slots); one barrier per K step: after it, every wave's row blocks of this step
//     have landed and the slot of the step before is free.
//   - Only the row blocks that hold rows are loaded and multiplied (a compile-time count,
//     one instantiation per count, so the K loop has no branch).
// bf16 chunks hold 16 columns x 32 K, the MFMA operand as it is; int8 chunks 16 columns x
// 64 K (bytes 0-7 the first 32-K half), widened to bf16 in registers; int4 chunks 16
// columns x 128 K (one scale group), unpacked as q + 136, with 136 * sum(a) taken off per
// group through the MFMA accumulator's starting value.
#include <type_traits>

#include "common.h"

namespace moe {
namespace {

constexpr int kNW = 4;                 // waves per workgroup
constexpr int kThreads = kNW * kWave;
constexpr int kGN = 4, kGNAll = 6;     // column tiles per group (see decode_tile_at)
constexpr int kChunk = 32;             // tiles dealt to the XCDs in chunks

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma16(const void* src, u32x4* lds_block) {
    __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_block, 16, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm_le() {
    static_assert(N >= 0 && N < 64, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t i8x2_bf16(uint32_t w, int sh) {
    const float f0 = (float)(int)(int8_t)(w >> sh);
    const float f1 = (float)(int)(int8_t)(w >> (sh + 8));
    // the high halves of the two fp32 patterns (exact for |q| <= 128), by one byte permute
    return __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
}

template <bool NT>
__device__ __forceinline__ u32x4 load_w(const u32x4* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

// K steps in flight per wave for MA row blocks of a tile of MB: as many as the registers
// left beside the accumulators hold (two waves per SIMD: 256 registers a wave; bf16 160-row
// tiles: 3)
template <int WQ>
__host__ __device__ constexpr int ring_depth(int MA, int MB) {
    return WQ == kWBf16 ? (MB > 8 ? 3 : 4) : WQ == kWI4 ? (MB > 4 ? 3 : MA <= 2 ? 4 : 3) : (MA <= 4 ? 4 : MA <= 6 ? 3 : 2);
}

// LDS of the K loop: (R + 1) slots of MA * KH 1 KB blocks, the most over MA <= MB
template <int WQ>
__host__ __device__ constexpr int ring_blocks(int MB) {
    int m = 0;
    for (int ma = 1; ma <= MB; ++ma) {
        const int b = (ring_depth<WQ>(ma, MB) + 1) * ma * (WQ == kWI4 ? 4 : WQ == kWI8 ? 2 : 1);
        m = b > m ? b : m;
    }
    return m;
}

// MB: 16-row blocks per tile (a.bm = 16 MB); WQ: kWBf16, kWI8 or kWI4; NBW: 16-column
// weight blocks per wave (4; 2 for the int8 down projection of experts with few rows)
template <int MB, int WQ, bool UP, int NBW>
__global__ __launch_bounds__(kThreads, 2) void expert_tstream(GemmArgs a) {
    constexpr bool INT4 = WQ == kWI4, BF16 = WQ == kWBf16;
    constexpr int KSTEP = INT4 ? 128 : BF16 ? 32 : 64;  // K per weight chunk
    constexpr int KH = KSTEP / 32;          // 32-K row-block fragments per K step
    constexpr int BN = kNW * NBW * 16;      // columns per workgroup
    static_assert(NBW == 4 || (!UP && NBW == 2), "the up epilogue writes 32-column H blocks");

    const int K = UP ? a.d : a.F;
    const int N = UP ? 2 * a.F : a.d;
    const int NT_ = N / BN;
    const int S = UP ? 1 : a.ksplit;
    Tile tl;
    int split = 0;
    if (!decode_tile_split(a.tile_start, a.offsets, a.Et, NT_, NT_ <= kGNAll ? NT_ : kGN, MB * 16, S, tl, split,
                           kChunk))
        return;
    const int Kp = K / S;
    const int kbase = split * Kp;
    const int nsteps = Kp / KSTEP;
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform: scalar addressing
    const int nb0 = tl.n * (BN / 16) + wave * NBW;  // first owned column block

    extern __shared__ u32x4 lds[];  // [R + 1][MA * KH][64]; the epilogue's patches afterwards

    // weights: block nb's chunks are contiguous along K ([E][N/16][K/KSTEP][64][16 B])
    // (uniform bases, per-lane offsets: the addresses take scalar registers)
    const int KB = K / KSTEP;
    const u32x4* bbase = reinterpret_cast<const u32x4*>(UP ? a.wgu : a.wdn) +
                         ((size_t)tl.e * N * KB * 4 + (size_t)nb0 * KB * 64 + kbase / KSTEP * 64);
    // int4: the column scales, [E][K/128][N]; lane reads its column's
    const float* sbase = (UP ? a.s_gate : a.s_down) + ((size_t)tl.e * KB + kbase / KSTEP) * N + nb0 * 16;
    // row blocks: the padded operand in fragment order ([R/16][K/32][64][8]); tile g owns
    // row blocks g*MB .. g*MB + MB-1. Shared virtual experts past the first read the first
    // one's token rows (the same tokens in the same order).
    const int e0 = a.Et - a.kt + a.k;
    const int ga = (UP && tl.e > e0) ? tl.g - a.tile_start[tl.e] + a.tile_start[e0] : tl.g;
    const bf16_t* abase = (UP ? a.xp : a.h) + (((size_t)ga * MB * (K / 32) + kbase / 32) * 64 + lane) * 8;
    const int mb_act = (tl.rows + 15) / 16;

    f32x4 acc[MB][NBW];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NBW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint32_t nib_mask = 0x000F000Fu;  // int4 unpacking: held in a register (one v_and_or_b32 a pair)
    if constexpr (INT4) asm volatile("" : "+v"(nib_mask));

    // MA: row blocks holding rows (compile time); NT: non-temporal weight loads, when the
    // expert has one row tile (its weights are read once). AW: LDS-DMA loads per wave per
    // step (the MA * KH blocks dealt to the waves in turn; a wave past the last block
    // re-loads the last one, the same bytes to the same place, so that every wave makes the
    // same number of loads per step and one wait count fits all).
    auto kloop = [&](auto ma, auto nt) __attribute__((always_inline)) {
        constexpr int MA = decltype(ma)::value;
        constexpr bool NT = decltype(nt)::value;
        constexpr int R = ring_depth<WQ>(MA, MB);  // K steps in flight
        constexpr int NS = R + 1;              // LDS slots
        constexpr int SLOT = MA * KH;          // 1 KB blocks per slot
        constexpr int AW = (MA * KH + kNW - 1) / kNW;
        constexpr int X = NBW + (INT4 ? NBW : 0) + AW;  // vector memory loads per wave per step
        static_assert((R - 1) * X < 64, "wait count");
        size_t aoff[AW];
        int aslot[AW];
#pragma unroll
        for (int i = 0; i < AW; ++i) {
            const int b = min(wave + kNW * i, MA * KH - 1);  // block = mb * KH + kh
            aoff[i] = ((size_t)(b / KH) * (K / 32) + b % KH) * 512;
            aslot[i] = b;
        }
        struct Regs {
            u32x4 b[NBW];
            float sc[NBW];
        };
        Regs ring[R];
        auto issue = [&](int s, Regs& rg, int slot) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < NBW; ++j) rg.b[j] = load_w<NT>(bbase + ((size_t)j * KB + s) * 64 + lane);
            if constexpr (INT4) {
#pragma unroll
                for (int j = 0; j < NBW; ++j) rg.sc[j] = sbase[(size_t)s * N + j * 16 + lane % 16];
            }
#pragma unroll
            for (int i = 0; i < AW; ++i)
                dma16(abase + aoff[i] + (size_t)s * KH * 512, lds + (size_t)(slot * SLOT + aslot[i]) * 64);
        };
        auto compute = [&](const Regs& rg, int slot) __attribute__((always_inline)) {
            const u32x4* la = lds + (size_t)slot * SLOT * 64 + lane;
            if constexpr (INT4) {
                // one scale group: the MFMAs of the rows' fragments against the constant -136
                // (bf16 0xC308) give -136 * the rows' sums over the group; the partial products
                // of the codes (read as q + 136) accumulate onto that, so each partial comes out
                // as sum(a * q), and acc += scale * partial is one FMA (8-expert 6144 x 16384
                // layer: 2-5% faster than subtracting the sums after, T = 48-4096). In passes
                // of at most two row blocks (one on 80-row tiles), each unpacking the weights
                // again, so that a pass's fragments and partials fit beside the accumulators
                // with three K steps in flight (64-row tiles: 1-3% over one pass with two
                // steps; 80-row tiles: T = 256-288 up projection 3-6% over two-block passes
                // with two steps, which also spilled).
                const bf16x8 kneg136 =
                    __builtin_bit_cast(bf16x8, u32x4{0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u});
                constexpr int MH = MB > 4 ? 1 : MA < 2 ? MA : 2;  // row blocks per pass
#pragma unroll
                for (int m0 = 0; m0 < MA; m0 += MH) {
                    bf16x8 af[MH][KH];
#pragma unroll
                    for (int i = 0; i < MH; ++i)
#pragma unroll
                        for (int kh = 0; kh < KH; ++kh)
                            if (m0 + i < MA) af[i][kh] = __builtin_bit_cast(bf16x8, la[((m0 + i) * KH + kh) * 64]);
                    // -136 * the rows' sums over the group: the partials' starting value
                    f32x4 zn[MH];
#pragma unroll
                    for (int i = 0; i < MH; ++i)
                        if (m0 + i < MA) {
                            zn[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int kh = 0; kh < KH; ++kh)
                                zn[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i][kh], kneg136, zn[i], 0, 0, 0);
                        }
                    f32x4 g[MH][NBW];
#pragma unroll
                    for (int kh = 0; kh < KH; ++kh) {
#pragma unroll
                        for (int j = 0; j < NBW; ++j) {
                            const uint32_t w = rg.b[j][kh];
                            const bf16x8 bw = __builtin_bit_cast(
                                bf16x8, u32x4{(w & nib_mask) | 0x43004300u, ((w >> 4) & nib_mask) | 0x43004300u,
                                              ((w >> 8) & nib_mask) | 0x43004300u, ((w >> 12) & nib_mask) | 0x43004300u});
#pragma unroll
                            for (int i = 0; i < MH; ++i)
                                if (m0 + i < MA)
                                    g[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i][kh], bw,
                                                                                      kh ? g[i][j] : zn[i], 0, 0, 0);
                        }
                    }
#pragma unroll
                    for (int j = 0; j < NBW; ++j)
#pragma unroll
                        for (int i = 0; i < MH; ++i)
                            if (m0 + i < MA)
#pragma unroll
                                for (int c = 0; c < 4; ++c)
                                    acc[m0 + i][j][c] = fmaf(rg.sc[j], g[i][j][c], acc[m0 + i][j][c]);
                }
            } else if constexpr (BF16) {
                // the weight chunks are the MFMA operands as they are; row block by row block
#pragma unroll
                for (int mb = 0; mb < MA; ++mb) {
                    const bf16x8 af = __builtin_bit_cast(bf16x8, la[mb * 64]);
#pragma unroll
                    for (int j = 0; j < NBW; ++j)
                        acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(bf16x8, rg.b[j]),
                                                                            acc[mb][j], 0, 0, 0);
                }
            } else {
                // per 32-K half: the four widened weight fragments, then row block by row block
                // (one row fragment live at a time)
#pragma unroll
                for (int kh = 0; kh < KH; ++kh) {
                    bf16x8 bw[NBW];
#pragma unroll
                    for (int j = 0; j < NBW; ++j) {
                        const uint32_t lo = kh ? rg.b[j].z : rg.b[j].x, hi = kh ? rg.b[j].w : rg.b[j].y;
                        bw[j] = __builtin_bit_cast(
                            bf16x8, u32x4{i8x2_bf16(lo, 0), i8x2_bf16(lo, 16), i8x2_bf16(hi, 0), i8x2_bf16(hi, 16)});
                    }
#pragma unroll
                    for (int mb = 0; mb < MA; ++mb) {
                        const bf16x8 af = __builtin_bit_cast(bf16x8, la[(mb * KH + kh) * 64]);
#pragma unroll
                        for (int j = 0; j < NBW; ++j)
                            acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bw[j], acc[mb][j], 0, 0, 0);
                    }
                }
            }
        };
        // step s: its loads have landed for this wave (wait), and for every wave (barrier,
        // which also frees the slot of step s-1); multiply; refill the ring entry and that
        // slot with step s + R (past the last step the last one is loaded again and never
        // used, so the loop has no branch)
        auto fence = []() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };
        auto step = [&](int s, Regs& rg) __attribute__((always_inline)) {
            wait_vm_le<(R - 1) * X>();
            lds_barrier();
            fence();
            compute(rg, s % NS);
            fence();
            issue(min(s + R, nsteps - 1), rg, (s + R) % NS);
            fence();
        };
#pragma unroll
        for (int u = 0; u < R; ++u) issue(min(u, nsteps - 1), ring[u], u);
        int s = 0;
        for (; s + R <= nsteps; s += R) {
#pragma unroll
            for (int u = 0; u < R; ++u) step(s + u, ring[u]);
        }
#pragma unroll
        for (int u = 0; u < R - 1; ++u)
            if (s + u < nsteps) step(s + u, ring[u]);
        wait_vm_le<0>();  // no LDS-DMA write may outlive the K loop
    };
    auto run = [&](auto nt) __attribute__((always_inline)) {
        if constexpr (MB == 5) {
            if (mb_act <= 1) kloop(std::integral_constant<int, 1>{}, nt);
            else if (mb_act == 2) kloop(std::integral_constant<int, 2>{}, nt);
            else if (mb_act == 3) kloop(std::integral_constant<int, 3>{}, nt);
            else if (mb_act == 4) kloop(std::integral_constant<int, 4>{}, nt);
            else kloop(std::integral_constant<int, 5>{}, nt);
        } else if constexpr (MB == 4) {
            if (mb_act <= 1) kloop(std::integral_constant<int, 1>{}, nt);
            else if (mb_act == 2) kloop(std::integral_constant<int, 2>{}, nt);
            else if (mb_act == 3) kloop(std::integral_constant<int, 3>{}, nt);
            else kloop(std::integral_constant<int, 4>{}, nt);
        } else if constexpr (MB == 10) {
            switch (mb_act) {
                case 0:
                case 1: kloop(std::integral_constant<int, 1>{}, nt); break;
                case 2: kloop(std::integral_constant<int, 2>{}, nt); break;
                case 3: kloop(std::integral_constant<int, 3>{}, nt); break;
                case 4: kloop(std::integral_constant<int, 4>{}, nt); break;
                case 5: kloop(std::integral_constant<int, 5>{}, nt); break;
                case 6: kloop(std::integral_constant<int, 6>{}, nt); break;
                case 7: kloop(std::integral_constant<int, 7>{}, nt); break;
                case 8: kloop(std::integral_constant<int, 8>{}, nt); break;
                case 9: kloop(std::integral_constant<int, 9>{}, nt); break;
                default: kloop(std::integral_constant<int, 10>{}, nt); break;
            }
        } else {
            static_assert(MB == 8, "row blocks per tile");
            switch (mb_act) {
                case 0:
                case 1: kloop(std::integral_constant<int, 1>{}, nt); break;
                case 2: kloop(std::integral_constant<int, 2>{}, nt); break;
                case 3: kloop(std::integral_constant<int, 3>{}, nt); break;
                case 4: kloop(std::integral_constant<int, 4>{}, nt); break;
                case 5: kloop(std::integral_constant<int, 5>{}, nt); break;
                case 6: kloop(std::integral_constant<int, 6>{}, nt); break;
                case 7: kloop(std::integral_constant<int, 7>{}, nt); break;
                default: kloop(std::integral_constant<int, 8>{}, nt); break;
            }
        }
    };
    if (a.tile_start[tl.e + 1] - a.tile_start[tl.e] == 1) run(std::true_type{});
    else run(std::false_type{});

    // ---- epilogue: the LDS-tiled kernels' output layouts, through a per-wave LDS patch (the
    // down projection with two column blocks per wave stores from the accumulators)
    const int col16 = lane % 16;
    const int rq = 4 * (lane / 16);
    __syncthreads();  // every wave is done with the row-block slots
    if constexpr (UP) {
        // H patch: 16 MB rows x 32 bf16 columns (the wave's two gate/up pairs); H goes out in
        // the down operand's fragment order (rows past the expert's last row inside a block
        // are zero: zero inputs)
        constexpr int PW = 8 * NBW;
        bf16_t* patch = reinterpret_cast<bf16_t*>(lds) + (size_t)wave * (16 * MB) * PW;
#pragma unroll
        for (int q = 0; q < NBW / 2; ++q) {
            float sg = 1.f, su = 1.f;
            if constexpr (WQ == kWI8) {
                const int f = (nb0 / 2 + q) * 16 + col16;
                sg = a.s_gate[(size_t)tl.e * a.F + f];
                su = a.s_up[(size_t)tl.e * a.F + f];
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float g = acc[mb][2 * q][i] * sg;
                    const float u = acc[mb][2 * q + 1][i] * su;
                    patch[(mb * 16 + rq + i) * PW + q * 16 + col16] = f32_to_bf16(silu(g) * u);
                }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the patch is written
        static_assert(PW == 32, "one 32-column H block per wave");
        const int fb = nb0 / 2 * 16 / 32;
        // H row blocks in the down projection's tiling (tiles of bm_h rows from
        // tile_start_h[e]): the block holding rows r0 .. r0+15 of expert e is
        // tile_start_h[e] * bm_h / 16 + r0 / 16 (with bm_h == bm, tile g's block mb). Only
        // blocks holding rows are written; the down kernel reads no others.
        const int hb0 = a.tile_start_h[tl.e] * (a.bm_h / 16) + tl.row0 / 16;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if (mb * 16 < tl.rows) {
                const u32x4 v =
                    *reinterpret_cast<const u32x4*>(patch + (mb * 16 + lane % 16) * PW + 8 * (lane / 16));
                const size_t blk = (size_t)(hb0 + mb) * (a.F / 32) + fb;
                *reinterpret_cast<u32x4*>(a.h + (blk * 64 + lane) * 8) = v;
            }
        }
    } else if constexpr (NBW == 2) {
        // fp32 partial rows straight from the accumulators (no LDS patch, so more workgroups
        // fit a CU): lane holds column lane%16 of each 16-column block, rows 4*(lane/16)+i,
        // one 64-byte row piece per block and row
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = mb * 16 + rq + i;
                if (r < tl.rows) {
                    const int cs = a.sorted_c[tl.seg0 + tl.row0 + r];
                    const int t = cs / a.kt, j = cs - t * a.kt;
                    const float wgt = j < a.k ? a.topk_w[(size_t)t * a.k + j] : a.gs[t];
                    float* orow = a.ow + ((size_t)cs * S + split) * a.d;
#pragma unroll
                    for (int jn = 0; jn < NBW; ++jn) {
                        const int n = (nb0 + jn) * 16 + col16;
                        float v = acc[mb][jn][i] * wgt;
                        if constexpr (WQ == kWI8) v *= a.s_down[(size_t)tl.e * a.d + n];
                        orow[n] = v;  // partial sum `split` of slot cs
                    }
                }
            }
    } else {
        // output patch: 16 MB rows x 32 fp32 columns, two 16-column blocks at a time
        float* patch = reinterpret_cast<float*>(lds) + (size_t)wave * (16 * MB) * 32;
#pragma unroll
        for (int nh = 0; nh < NBW / 2; ++nh) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) patch[(mb * 16 + rq + i) * 32 + j * 16 + col16] = acc[mb][2 * nh + j][i];
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
            const int n0 = (nb0 + 2 * nh) * 16;
            for (int c = lane; c < 16 * MB * 8; c += kWave) {
                const int r = c / 8, c4 = (c % 8) * 4;
                if (r < tl.rows) {
                    const int cs = a.sorted_c[tl.seg0 + tl.row0 + r];
                    const int t = cs / a.kt, j = cs - t * a.kt;
                    const float wgt = j < a.k ? a.topk_w[(size_t)t * a.k + j] : a.gs[t];
                    f32x4 v = *reinterpret_cast<const f32x4*>(patch + r * 32 + c4) * wgt;
                    if constexpr (WQ == kWI8) v *= *reinterpret_cast<const f32x4*>(a.s_down + (size_t)tl.e * a.d + n0 + c4);
                    // partial sum `split` of slot cs: row cs*S + split of the combine buffer
                    *reinterpret_cast<f32x4*>(a.ow + ((size_t)cs * S + split) * a.d + n0 + c4) = v;
                }
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // patch reads done before the next half overwrites it
        }
    }
}

template <int MB, int WQ, bool UP, int NBW>
hipError_t launch_r(const GemmArgs& a, hipStream_t s) {
    constexpr int KSTEP = WQ == kWI4 ? 128 : WQ == kWI8 ? 64 : 32;
    constexpr int BN = kNW * NBW * 16;
    constexpr size_t ring = (size_t)ring_blocks<WQ>(MB) * 1024;
    constexpr size_t patch = UP ? (size_t)kNW * 16 * MB * 32 * 2 : NBW == 4 ? (size_t)kNW * 16 * MB * 32 * 4 : 0;
    constexpr size_t lds_bytes = ring > patch ? ring : patch;
    static_assert(lds_bytes * (8 / kNW) <= 160 * 1024, "two waves per SIMD");
    const int N = UP ? 2 * a.F : a.d;
    const int S = UP ? 1 : a.ksplit;
    const int Kp = (UP ? a.d : a.F) / S;
    if (a.bm != MB * 16 || N % BN != 0 || Kp % KSTEP != 0 || Kp < KSTEP) return hipErrorInvalidValue;
    const int NT = N / BN;
    const int gn = NT <= kGNAll ? NT : kGN;
    const int NTp = (NT + gn - 1) / gn * gn;
    // the chunked deal needs the tile count rounded up to whole chunks per XCD
    const size_t blocks = (size_t)a.max_tiles * NTp * S + kXcds * kChunk;
    const dim3 grid((unsigned)((blocks + kXcds - 1) / kXcds * kXcds));
    auto kern = expert_tstream<MB, WQ, UP, NBW>;
    static bool attr_set = false;  // one-time opt-in above the default dynamic LDS limit
    if (!attr_set) {
        const hipError_t e =
            hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds_bytes, s, a);
    return hipGetLastError();
}

template <int WQ, bool UP>
hipError_t launch_w(const GemmArgs& a, hipStream_t s) {
    // The int8 down projection while the experts average at most 64 rows: two column blocks
    // per wave (128 registers: four workgroups per CU with 64-row tiles, three with 128-row
    // ones; 8-expert 6144 x 16384 layer: T = 64 down 166 -> 140 us, layer 451 -> 429 us;
    // T = 192 519 against 528 us). With more rows, or int4 weights, the doubled row-fragment
    // reads per weight byte cost more than the waves gain (int8 T = 384: 671 -> 688 us, T =
    // 1024 down 493 -> 594 us).
    if constexpr (WQ == kWBf16) {
        // 128-row tiles, or 160 rows when the experts average 97-128 (one tile for most)
        if (a.bm == 128) return launch_r<8, WQ, UP, 4>(a, s);
        if (a.bm == 160) return launch_r<10, WQ, UP, 4>(a, s);
    } else if constexpr (WQ == kWI4) {
        if constexpr (UP) {  // 80-row tiles: up projection only (its down projection tiles by 64, bm_h)
            if (a.bm == 80) return launch_r<5, WQ, UP, 4>(a, s);
        }
        if (a.bm == 64) return launch_r<4, WQ, UP, 4>(a, s);
    } else {
        if constexpr (!UP) {
            if (tstream_narrow_down(a.T, a.k, a.Et)) {
                if (a.bm == 128) return launch_r<8, WQ, UP, 2>(a, s);
                if (a.bm == 64) return launch_r<4, WQ, UP, 2>(a, s);
            }
        }
        if (a.bm == 128) return launch_r<8, WQ, UP, 4>(a, s);
        if (a.bm == 64) return launch_r<4, WQ, UP, 4>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_expert_up_tstream(const GemmArgs& a, int wq, hipStream_t s) {
    if (wq == kWBf16) return launch_w<kWBf16, true>(a, s);
    if (wq == kWI8) return launch_w<kWI8, true>(a, s);
    if (wq == kWI4) return launch_w<kWI4, true>(a, s);
    return hipErrorInvalidValue;
}

hipError_t launch_expert_down_tstream(const GemmArgs& a, int wq, hipStream_t s) {
    if (wq == kWBf16) return launch_w<kWBf16, false>(a, s);
    if (wq == kWI8) return launch_w<kWI8, false>(a, s);
    if (wq == kWI4) return launch_w<kWI4, false>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace moe
