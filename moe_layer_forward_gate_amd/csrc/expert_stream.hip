// Expert compute for small batches (decode): weight-streaming grouped GEMMs.
//
// With a handful of tokens the expert weights are the only real traffic
// ([hotelren §2.1]: the bottleneck is moving data, not arithmetic), so this path
// is built to stream each active expert's packed weights from HBM exactly once
// at full width, with every weight byte fetched by exactly one wave:
//   - every wave owns NBW 16-column weight blocks and a K range; it reads them
//     as contiguous 1 KB fragment blocks (16 B per lane: 32 bf16, 64 int8 or 128
//     int4 K rows of one column) straight into MFMA operand registers, U K-steps
//     at a time so many loads are in flight, as non-temporal loads when each
//     weight byte is read once per forward (keeping it out of the caches'
//     working set streams ~10% faster);
//   - the few token rows (<= 16*MB) come in as MFMA A fragments from L2;
//   - the down projection splits K over S workgroups when the active experts
//     alone would leave the GPU idle; each split writes its own partial row of
//     the combine buffer (row c*S + s) and the Gather pass adds them, so the
//     result does not depend on scheduling.
// Work item = (active expert, group of 4*NBW column blocks, K split); experts
// without rows get no work items (the item count is read from the scatter's tile
// table on the device).
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr size_t kAStageBytes = 32 * 1024;  // LDS for a work item's token rows (see expert_stream)

__device__ __forceinline__ uint32_t i8x2_bf16(uint32_t w, int sh) {
    const float f0 = (float)(int)(int8_t)(w >> sh);
    const float f1 = (float)(int)(int8_t)(w >> (sh + 8));
    // the high halves of the two fp32 patterns (exact: |q| <= 128 has at most 8 significant
    // bits), picked by one byte permute: bytes 2-3 of f0, then bytes 2-3 of f1
    return __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
}

// int4 codes (q + 8, 4 bits) to bf16 pairs: a code u placed in the low mantissa bits of
// 0x4300 (bf16 128.0, whose unit in the last place is 1) reads as 128 + u = q + 136, so
// one mask-and-or turns two codes into two exact bf16 values; the products' excess
// 136 * sum(a) over the group is taken off after the MFMAs. A lane's 32-bit word holds
// K rows 2i in nibble i and 2i+1 in nibble i+4 (i < 4), so word >> 4i yields the pair
// (2i, 2i+1) in the two bf16 halves.
// The caller passes the nibble mask in a register (opaque to the compiler), so that each
// pair is one v_and_or_b32 with the bf16 pattern as its literal (a VOP3 instruction
// reads at most one literal or scalar).
__device__ __forceinline__ u32x4 i4x8_bf16(uint32_t w, uint32_t m) {
    return u32x4{(w & m) | 0x43004300u, ((w >> 4) & m) | 0x43004300u, ((w >> 8) & m) | 0x43004300u,
                 ((w >> 12) & m) | 0x43004300u};
}

template <bool NT>
__device__ __forceinline__ u32x4 load_w(const u32x4* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

// WQ: weight kind (kWBf16, kWI8, kWI4); NT: the weights are loaded non-temporally
template <int MB, int NBW, int WQ, bool UP, int U, bool NT, bool AL>
__global__ __launch_bounds__(kThreads) void expert_stream(GemmArgs a, int S) {
    constexpr bool INT8 = WQ == kWI8;
    constexpr bool INT4 = WQ == kWI4;
    // K covered by one 16-byte weight chunk per lane (an int4 chunk is one scale group)
    constexpr int KSTEP = INT4 ? 128 : INT8 ? 64 : 32;
    constexpr int KH = KSTEP / 32;
    const int K = UP ? a.d : a.F;
    const int N = UP ? 2 * a.F : a.d;
    const int NG = N / (16 * NBW * 4);  // column groups per expert
    // ---- work item
    const int total = a.tile_start[a.Et] * NG * S;
    const int L = blockIdx.x;
    if (L >= total) return;
    const int tile = L / (NG * S);
    const int rem = L - tile * NG * S;
    const int ng = rem / S, split = rem - (rem / S) * S;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    int c = 0;
    for (int j0 = 0; j0 <= a.Et; j0 += kWave) {
        const int j = j0 + lane;
        c += __popcll(__ballot(j <= a.Et && a.tile_start[j] <= tile));
    }
    const int e = c - 1;
    const int seg0 = a.offsets[e] + (tile - a.tile_start[e]) * a.bm;
    const int rows = min(a.bm, a.offsets[e + 1] - seg0);
    const int mb_act = (rows + 15) / 16;  // <= MB by construction of the launch

    const int Kp = K / S;
    const int kbase = split * Kp;
    const int nsteps = Kp / KSTEP;
    const int nb0 = (ng * 4 + wave) * NBW;

    // weight stream of each owned column block: contiguous 1 KB chunks along K
    const u32x4* bptr[NBW];
    const float* sptr[NBW];  // int4: the group scales of the lane's column, one per K step
    {
        const int KB = K / KSTEP;
        // one expert: N * K / KSTEP blocks of 1 KB (64 chunks of 16 bytes)
        const u32x4* wb = reinterpret_cast<const u32x4*>(UP ? a.wgu : a.wdn) + (size_t)e * N * KB * 4;
#pragma unroll
        for (int j = 0; j < NBW; ++j) bptr[j] = wb + ((size_t)(nb0 + j) * KB + kbase / KSTEP) * 64 + lane;
#pragma unroll
        for (int j = 0; j < NBW; ++j)
            sptr[j] = (UP ? a.s_gate : a.s_down) + ((size_t)e * KB + kbase / KSTEP) * N + (nb0 + j) * 16 + lane % 16;
    }
    // token rows as A fragments: lane holds row 16*mb + lane%16, K 8*(lane/16)..+7 (rows past
    // the work item's last row repeat its first: their outputs are never stored)
    const bf16_t* aptr[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int r = mb * 16 + lane % 16;
        const int p = seg0 + (r < rows ? r : 0);
        const bf16_t* base = UP ? a.x + (size_t)(a.sorted_c[p] / a.kt) * a.d : a.h + (size_t)p * a.F;
        aptr[mb] = base + kbase + 8 * (lane / 16);
    }
    // AL (int4, one row block, a few rows): the work item's rows over its K range are copied
    // to LDS once, and the fragments are read from there, so the weight stream has more of
    // the vector memory path (from global memory the four waves read the same rows, and 15
    // of a fragment's 16 rows repeat the first when a tile holds one row)
    extern __shared__ u32x4 arow[];  // AL: [rows][Kp / 8] 16-byte chunks
    const int cpr = Kp / 8;
    if constexpr (AL) {
        static_assert(MB == 1, "LDS-staged rows: one row block");
        for (int c = threadIdx.x; c < rows * cpr; c += kThreads) {
            const int r = c / cpr, q = c - r * cpr;
            const bf16_t* base = UP ? a.x + (size_t)(a.sorted_c[seg0 + r] / a.kt) * a.d : a.h + (size_t)(seg0 + r) * a.F;
            arow[c] = *reinterpret_cast<const u32x4*>(base + kbase + 8 * q);
        }
        __syncthreads();
    }
    const int arr = lane % 16 < rows ? lane % 16 : 0;  // AL: the LDS row this lane reads
    auto a_frag = [&](int mb, int s, int kh) __attribute__((always_inline)) -> u32x4 {
        if constexpr (AL) return arow[arr * cpr + (s * KSTEP + kh * 32) / 8 + lane / 16];
        else return *reinterpret_cast<const u32x4*>(aptr[mb] + s * KSTEP + kh * 32);
    };

    uint32_t nib_mask = 0x000F000Fu;  // int4 unpacking (see i4x8_bf16)
    if constexpr (INT4) asm volatile("" : "+v"(nib_mask));

    f32x4 acc[MB][NBW];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NBW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The K loop runs with the number of row blocks that hold rows (MA <= MB) fixed at
    // compile time and no other branch in its steady state: a branch inside it makes the
    // compiler wait for every load in flight (vmcnt(0)) before the next round's loads and
    // again before the MFMAs, which drains the two-round pipeline every round.
    auto kloop = [&](auto ma) __attribute__((always_inline)) {
        constexpr int MA = decltype(ma)::value;
        auto step = [&](const u32x4 (&bb)[NBW], const u32x4 (&aa)[MB][KH], const float (&sc)[NBW])
                        __attribute__((always_inline)) {
            if constexpr (INT4) {
                // one scale group: the MFMAs of the token fragments against the constant -136
                // give -136 * the rows' sums over the group, the partial products of the codes
                // (read as q + 136) accumulate onto that, so each partial comes out as
                // sum(a * q), and acc += scale * partial is one FMA
                const bf16x8 kneg136 =
                    __builtin_bit_cast(bf16x8, u32x4{0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u});
                f32x4 zn[MA], g[NBW][MA];
#pragma unroll
                for (int mb = 0; mb < MA; ++mb) {
                    zn[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kh = 0; kh < KH; ++kh)
                        zn[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, aa[mb][kh]), kneg136,
                                                                         zn[mb], 0, 0, 0);
                }
#pragma unroll
                for (int kh = 0; kh < KH; ++kh) {
#pragma unroll
                    for (int j = 0; j < NBW; ++j) {
                        const bf16x8 bw = __builtin_bit_cast(bf16x8, i4x8_bf16(bb[j][kh], nib_mask));
#pragma unroll
                        for (int mb = 0; mb < MA; ++mb)
                            g[j][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8, aa[mb][kh]), bw, kh ? g[j][mb] : zn[mb], 0, 0, 0);
                    }
                }
#pragma unroll
                for (int j = 0; j < NBW; ++j)
#pragma unroll
                    for (int mb = 0; mb < MA; ++mb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[mb][j][i] = fmaf(sc[j], g[j][mb][i], acc[mb][j][i]);
                return;
            }
#pragma unroll
            for (int kh = 0; kh < KH; ++kh)
#pragma unroll
                for (int j = 0; j < NBW; ++j) {
                    u32x4 bw;
                    if constexpr (INT8) {
                        const uint32_t lo = kh ? bb[j].z : bb[j].x, hi = kh ? bb[j].w : bb[j].y;
                        bw = u32x4{i8x2_bf16(lo, 0), i8x2_bf16(lo, 16), i8x2_bf16(hi, 0), i8x2_bf16(hi, 16)};
                    } else {
                        bw = bb[j];
                    }
#pragma unroll
                    for (int mb = 0; mb < MA; ++mb)
                        acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, aa[mb][kh]), __builtin_bit_cast(bf16x8, bw), acc[mb][j], 0,
                            0, 0);
                }
        };

        // rounds of U K-steps, double-buffered: the loads of round r+1 are issued before the
        // MFMAs of round r, so every wave always has a round of weight loads in flight
        struct Round {
            u32x4 bb[U][NBW];
            u32x4 aa[U][MB][KH];
            float sc[U][NBW];  // int4 only
        };
        auto load_round = [&](Round& R, int s0) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int j = 0; j < NBW; ++j) R.bb[u][j] = load_w<NT>(&bptr[j][(size_t)(s0 + u) * 64]);
            if constexpr (INT4) {
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int j = 0; j < NBW; ++j) R.sc[u][j] = sptr[j][(size_t)(s0 + u) * N];
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int mb = 0; mb < MA; ++mb)
#pragma unroll
                    for (int kh = 0; kh < KH; ++kh)
                        R.aa[u][mb][kh] = a_frag(mb, s0 + u, kh);
        };
        auto compute_round = [&](const Round& R) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < U; ++u) step(R.bb[u], R.aa[u], R.sc[u]);
        };
        // the scheduler may not move a round's loads past the MFMAs of the round before
        // (left to itself it sinks loads to shorten register lifetimes, and the waits
        // then drain the queue)
        auto fence = []() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };
        const int nround = nsteps / U;
        if (nround > 0) {
            Round r0, r1;
            load_round(r0, 0);
            int r = 0;
            for (; r + 2 < nround; r += 2) {  // steady state: two rounds always in flight
                fence();
                load_round(r1, (r + 1) * U);
                fence();
                compute_round(r0);
                fence();
                load_round(r0, (r + 2) * U);
                fence();
                compute_round(r1);
            }
            fence();
            if (nround - r == 2) {
                load_round(r1, (r + 1) * U);
                fence();
                compute_round(r0);
                compute_round(r1);
            } else {
                compute_round(r0);
            }
        }
        for (int s = nround * U; s < nsteps; ++s) {
            u32x4 bb[NBW];
            u32x4 aa[MB][KH];
            float sc[NBW] = {};
#pragma unroll
            for (int j = 0; j < NBW; ++j) bb[j] = load_w<NT>(&bptr[j][(size_t)s * 64]);
            if constexpr (INT4) {
#pragma unroll
                for (int j = 0; j < NBW; ++j) sc[j] = sptr[j][(size_t)s * N];
            }
#pragma unroll
            for (int mb = 0; mb < MA; ++mb)
#pragma unroll
                for (int kh = 0; kh < KH; ++kh)
                    aa[mb][kh] = a_frag(mb, s, kh);
            step(bb, aa, sc);
        }
    };
    // row blocks holding rows: 1 .. MB (a work item always holds at least one row)
    if constexpr (MB == 1) {
        kloop(std::integral_constant<int, 1>{});
    } else if constexpr (MB == 2) {
        if (mb_act == 1) kloop(std::integral_constant<int, 1>{});
        else kloop(std::integral_constant<int, 2>{});
    } else {
        static_assert(MB == 4, "row blocks per work item");
        if (mb_act == 1) kloop(std::integral_constant<int, 1>{});
        else if (mb_act == 2) kloop(std::integral_constant<int, 2>{});
        else if (mb_act == 3) kloop(std::integral_constant<int, 3>{});
        else kloop(std::integral_constant<int, 4>{});
    }

    // ---- epilogue (same fragment layout as the prefill kernels)
    const int col16 = lane % 16, rq = 4 * (lane / 16);
    if constexpr (UP) {
#pragma unroll
        for (int q = 0; q < NBW / 2; ++q) {
            const int f = (nb0 / 2 + q) * 16 + col16;
            float sg = 1.f, su = 1.f;
            if constexpr (INT8) {
                sg = a.s_gate[(size_t)e * a.F + f];
                su = a.s_up[(size_t)e * a.F + f];
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = mb * 16 + rq + i;
                    if (r < rows) {
                        const float g = acc[mb][2 * q][i] * sg, u = acc[mb][2 * q + 1][i] * su;
                        a.h[(size_t)(seg0 + r) * a.F + f] = f32_to_bf16(silu(g) * u);
                    }
                }
        }
    } else {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = mb * 16 + rq + i;
                if (r < rows) {
                    const int cs = a.sorted_c[seg0 + r];
                    const int t = cs / a.kt, j = cs - t * a.kt;
                    const float wgt = j < a.k ? a.topk_w[(size_t)t * a.k + j] : a.gs[t];
                    float* orow = a.ow + ((size_t)cs * S + split) * a.d;
#pragma unroll
                    for (int jn = 0; jn < NBW; ++jn) {
                        const int n = (nb0 + jn) * 16 + col16;
                        float v = acc[mb][jn][i] * wgt;
                        if constexpr (INT8) v *= a.s_down[(size_t)e * a.d + n];
                        orow[n] = v;
                    }
                }
            }
    }
}

template <int MB, int NBW, int WQ, bool UP>
hipError_t launch_nbw(const GemmArgs& a, int S, hipStream_t s) {
    // K-steps per round (two rounds are in flight per wave); an int4 step holds four
    // 32-K token fragments per row block, so wide row tiles take one step per round. The
    // bf16 up projection of one-block row tiles takes 8 (222 registers, two waves per SIMD,
    // against 126 and three at 4: its grid has too few waves to hide HBM latency otherwise;
    // 8-expert layer T = 1 up 80.9 -> 79.9 us, T = 8 270.5 -> 267.8 us). It runs without a K
    // split, so its d / 32 steps are whole rounds when d % 256 == 0 (other widths finish in
    // the per-step loop after the rounds); int8 with 3 steps: no change.
    constexpr int U = WQ == kWI4 ? (MB <= 1 ? 2 : 1) : WQ == kWI8 ? 2 : (MB <= 1 && UP ? 8 : MB <= 2 ? 4 : 2);
    constexpr int KSTEP = WQ == kWI4 ? 128 : WQ == kWI8 ? 64 : 32;
    const int N = UP ? 2 * a.F : a.d;
    if (((UP ? a.d : a.F) / S) % KSTEP != 0) return hipErrorInvalidValue;  // whole K steps per split
    if (N % (16 * NBW * 4) != 0) return hipErrorInvalidValue;             // whole column groups
    const int NG = N / (16 * NBW * 4);
    dim3 grid((unsigned)((size_t)a.max_tiles * NG * S));
    // non-temporal weight loads when each expert's weights are read by one row tile; an int4
    // layer whose busiest expert needs several 32-row tiles streams them once per tile and
    // keeps them cached
    // int4 one-row-block tiles whose rows over the K range fit kAStageBytes take them from
    // LDS (an int4 K step reads four token fragments a block; int4 T = 1 79.4 -> 76.8 us).
    // bf16 and int8 keep reading them from global memory: the copy and its barrier come
    // before their weight stream starts (T = 1: 125.2 -> 127.8 and 109.3 -> 112.4 us). A
    // tile holds at most min(bm, T * k) rows (a given routing may repeat an expert within a
    // token; a shared slice holds T rows).
    const size_t astage = (size_t)std::min(a.bm, a.T * a.k) * ((UP ? a.d : a.F) / S) * 2;
    if constexpr (MB == 1 && WQ == kWI4) {
        if (astage <= kAStageBytes) {
            if (WQ != kWI4 || a.weights_once)
                hipLaunchKernelGGL((expert_stream<MB, NBW, WQ, UP, U, true, true>), grid, dim3(kThreads), astage, s, a,
                                   S);
            else if constexpr (WQ == kWI4)
                hipLaunchKernelGGL((expert_stream<MB, NBW, WQ, UP, U, false, true>), grid, dim3(kThreads), astage, s,
                                   a, S);
            return hipGetLastError();
        }
    }
    if (WQ != kWI4 || a.weights_once)
        hipLaunchKernelGGL((expert_stream<MB, NBW, WQ, UP, U, true, false>), grid, dim3(kThreads), 0, s, a, S);
    else if constexpr (WQ == kWI4)
        hipLaunchKernelGGL((expert_stream<MB, NBW, WQ, UP, U, false, false>), grid, dim3(kThreads), 0, s, a, S);
    return hipGetLastError();
}

template <int MB, int WQ, bool UP>
hipError_t launch_mb(const GemmArgs& a, int S, hipStream_t s) {
    // int4: four column blocks per wave (the token fragments and the group sums serve
    // twice the weights) when that still leaves ~4 workgroups per CU and the row tile is
    // narrow enough for the registers
    if constexpr (WQ == kWI4 && MB <= 2) {
        const int N = UP ? 2 * a.F : a.d;
        if (N % 256 == 0 && (size_t)a.max_tiles * (N / 256) * S >= 1024) return launch_nbw<MB, 4, WQ, UP>(a, S, s);
    }
    return launch_nbw<MB, 2, WQ, UP>(a, S, s);
}

template <int WQ, bool UP>
hipError_t launch_t(const GemmArgs& a, int S, hipStream_t s) {
    switch ((a.bm + 15) / 16) {
        case 1: return launch_mb<1, WQ, UP>(a, S, s);
        case 2: return launch_mb<2, WQ, UP>(a, S, s);
        case 3:
        case 4:
            if constexpr (WQ == kWI4) return hipErrorInvalidValue;  // int4 row tiles are at most 32 rows
            else return launch_mb<4, WQ, UP>(a, S, s);
        default: return hipErrorInvalidValue;
    }
}

template <bool UP>
hipError_t launch_kind(const GemmArgs& a, int wq, int S, hipStream_t s) {
    switch (wq) {
        case kWBf16: return launch_t<kWBf16, UP>(a, S, s);
        case kWI8: return launch_t<kWI8, UP>(a, S, s);
        case kWI4: return launch_t<kWI4, UP>(a, S, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_expert_up_stream(const GemmArgs& a, int wq, hipStream_t s) { return launch_kind<true>(a, wq, 1, s); }

hipError_t launch_expert_down_stream(const GemmArgs& a, int wq, hipStream_t s) {
    return launch_kind<false>(a, wq, a.ksplit, s);
}

}  // namespace moe
