// Gate: router logits (fp32), wavefront top-k, softmax over the chosen logits and
// the shared-expert sigmoid gate.
//
// [hotelren §3.2] the router is a linear projection of each token; [0539edu §2.1]
// the gate yields one logit per expert and the top-k are kept; [mhpq §3.2] the
// running-maximum selection uses a strict greater-than, so equal logits keep the
// lower expert id and slot 0 holds the maximum; [pptc §2.1] the top-k is found
// inside one wavefront with cross-lane shuffles and no block-wide barrier.
//
// Three logit paths share the same top-k code:
//   - gate_rowdot (T <= 64): one workgroup per token; the 256 threads split K and
//     take the router rows eight at a time, so every load of the token and of the
//     router weights is in flight at once (decode: latency is what counts);
//   - gate_mfma_part + gate_mfma_finish (T > 64, bf16 tokens): 128 tokens x a K
//     slice per workgroup on bf16 MFMA, router and token fragments staged in LDS;
//     the slices' partial logits are added in order by the finish launch. The
//     fp32 router weight is carried as three bf16 planes w = hi + mid + lo (an
//     exact split: each plane takes the next 8 significant bits), and a bf16
//     token times a bf16 plane is exact in the fp32 accumulator, so the three
//     products summed in fp32 give the fp32 router GEMM;
//   - gate_tiled (T > 64, fp32 tokens): LDS-tiled fp32 FMA.
#include <type_traits>

#include "common.h"
#include "scatter.h"
#include "topk.h"

namespace moe {
namespace {

template <typename XT>
__device__ __forceinline__ void load8(const XT* p, float* v);
template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float* v) {
    uint4 q = *reinterpret_cast<const uint4*>(p);
    uint32_t a[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(a[i] << 16);
        v[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
    }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
    float4 a = reinterpret_cast<const float4*>(p)[0];
    float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// ---------------------------------------------------------------- decode path
// grid = T workgroups of 256 threads. Thread tid owns K chunks tid*8 + 2048*c
// (c < XC, d <= 2048*XC); router rows are taken 8 at a time, each thread forms 8
// partial dots, a wave butterfly folds them and the 4 wave partials meet in LDS.
// The token's chunks stay packed until the multiply-adds, so the router loads are
// issued without waiting for them (a decode step is a chain of memory latencies).
constexpr int kRowXC = 4;  // d <= 8192
template <typename XT, int XC>
__global__ __launch_bounds__(256) void gate_rowdot(const XT* __restrict__ x, const float* __restrict__ wr_t,
                                                   const float* __restrict__ bias, int d, int E, int Ec, int k,
                                                   int gflags, int32_t* __restrict__ idx,
                                                   float* __restrict__ w, float* __restrict__ gs) {
    __shared__ float part[4][kMaxExperts + 8];
    __shared__ float logits[kMaxExperts + 8];
    const int t = blockIdx.x;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const XT* xr = x + (size_t)t * d;
    // every load is unconditional (a chunk past d reads a valid address and is dropped)
    float wv[XC][8][8];
    auto load_group = [&](int e0) {
#pragma unroll
        for (int c = 0; c < XC; ++c) {
            const int kk = tid * 8 + 2048 * c;
            const int kc = kk < d ? kk : 0;
#pragma unroll
            for (int g = 0; g < 8; ++g) {
                const int e = e0 + g < Ec ? e0 + g : 0;
                load8<float>(wr_t + (size_t)e * d + kc, wv[c][g]);
            }
        }
    };
    load_group(0);  // requested before the token's chunks, so both are in flight together
    constexpr int XQ = sizeof(XT) / 2;  // 16-byte chunks per 8 elements
    u32x4 xq[XC][XQ];
#pragma unroll
    for (int c = 0; c < XC; ++c) {
        const int kk = tid * 8 + 2048 * c;
        const u32x4* p = reinterpret_cast<const u32x4*>(xr + (kk < d ? kk : 0));
#pragma unroll
        for (int q = 0; q < XQ; ++q) xq[c][q] = p[q];
    }
    auto xval = [&](int c, int v) {
        if constexpr (XQ == 1) {
            const uint32_t u = xq[c][0][v / 2];
            return __uint_as_float((v & 1) ? (u & 0xFFFF0000u) : (u << 16));
        } else {
            return __uint_as_float(xq[c][v / 4][v % 4]);
        }
    };
    for (int e0 = 0; e0 < Ec; e0 += 8) {
        if (e0 > 0) load_group(e0);
        float acc[8];
#pragma unroll
        for (int g = 0; g < 8; ++g) acc[g] = 0.0f;
#pragma unroll
        for (int c = 0; c < XC; ++c) {
            const bool ok = tid * 8 + 2048 * c < d;
#pragma unroll
            for (int g = 0; g < 8; ++g)
#pragma unroll
                for (int v = 0; v < 8; ++v) acc[g] = fmaf(ok ? xval(c, v) : 0.0f, wv[c][g][v], acc[g]);
        }
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            const float sum = wave_sum(acc[g]);
            if (lane == 0 && e0 + g < Ec) part[wave][e0 + g] = sum;
        }
    }
    __syncthreads();
    if (tid < Ec) {
        const float b = (bias && tid < E) ? bias[tid] : 0.0f;
        logits[tid] = (part[0][tid] + part[1][tid]) + (part[2][tid] + part[3][tid]) + b;
    }
    __syncthreads();
    if (wave == 0) wave_topk_write(logits, E, k, gflags, t, idx, w, gs);
}

// ---------------------------------------------------------------- prefill path, bf16 tokens
// Two launches. gate_mfma_part: workgroup (tile of 64*TPW tokens, K slice) of four waves,
// wave w owning the tile's token blocks w*TPW .. w*TPW+TPW-1 (16 tokens each). Every K step
// of 32 brings the three router planes' blocks (3*NB of 1 KB, fragment order) and the
// tile's token fragments (4*TPW blocks of 16 rows x 32 K, gathered from the token rows)
// into LDS by LDS-DMA, four steps in flight, so each router block is read once per 64*TPW
// tokens and shared by the four waves (a workgroup per 16 or 32 tokens, each re-reading
// the whole router, made the router reads the gate's cost). Each wave multiplies its
// token blocks by the three planes (smallest first) and writes the slice's partial logits
// to part[slice][token][NC]. gate_mfma_finish: one wave per token adds the slices in order
// and the bias, then runs the top-k.
constexpr int kGateTPW = 2;         // token blocks per wave: 128 tokens per workgroup
constexpr int kGateStages = 4;
constexpr int kGateMinSteps = 4;    // K steps per slice at least (pipeline fill)

__host__ __device__ __forceinline__ int gate_mfma_tiles(int T) { return (T + 64 * kGateTPW - 1) / (64 * kGateTPW); }
// K slices of kps steps each: enough (token tile, slice) workgroups to cover the CUs, each
// slice at least kGateMinSteps K steps (but for K under that); the count is taken from kps so
// that every slice holds at least one step: (slices - 1) * kps < KS
__host__ __device__ __forceinline__ int gate_mfma_kps(int T, int d) {
    const int KS = d / 32;
    const int want = (256 + gate_mfma_tiles(T) - 1) / gate_mfma_tiles(T);
    const int most = KS / kGateMinSteps > 0 ? KS / kGateMinSteps : 1;
    const int S = want < most ? want : most;
    return (KS + S - 1) / S;
}
__host__ __device__ __forceinline__ int gate_mfma_slices(int T, int d) {
    const int kps = gate_mfma_kps(T, d);
    return (d / 32 + kps - 1) / kps;
}

// one 16-byte LDS-DMA load per lane: LDS[block + 16*lane] = *src (block is wave-uniform)
__device__ __forceinline__ void gate_dma16(const void* src, u32x4* lds_block) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_block, 16, 0, 0);
}

// s_waitcnt vmcnt <= N and lgkmcnt 0 (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8): this wave's loads but the last N have landed and its LDS reads are done
template <int N>
__device__ __forceinline__ void gate_wait_vm_lds() {
    static_assert(N >= 0 && N < 64, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

template <int NB>
__global__ __launch_bounds__(512, 1) void gate_mfma_part(const bf16_t* __restrict__ x, const u32x4* __restrict__ planes,
                                                        int T, int d, int kps, float* __restrict__ part) {
    constexpr int NW = 8;                      // waves: token group w % 4, column half w / 4
    constexpr int TPW = kGateTPW;
    constexpr int NB0 = (NB + 1) / 2;          // column blocks of the first half (the second takes the rest)
    constexpr int NBL = 3 * NB;                // router blocks per K step
    constexpr int LB = (NBL + NW - 1) / NW;    // router block loads per wave per step
    constexpr int ABLK = 4 * TPW;              // token blocks per stage
    static_assert(ABLK % NW == 0, "token blocks: a whole number per wave");
    constexpr int LA = ABLK / NW;              // token block loads per wave per step
    constexpr int L = LA + LB;                 // LDS-DMA loads per wave per step
    constexpr int STAGE = ABLK + NW * LB;      // 1 KB blocks per stage
    constexpr int STAGES = kGateStages;
    constexpr int NC = NB * 16;
    extern __shared__ u32x4 lds[];             // [STAGES][STAGE][64 lanes]
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int tg = wave % 4, ch = wave / 4;
    const int KS = d / 32;
    const int ks0 = blockIdx.y * kps;
    const int nsteps = min(KS, ks0 + kps) - ks0;
    const int t0 = blockIdx.x * 64 * TPW;
    // token fragment loads: wave w fills token blocks w*LA .. (block b holds tokens
    // t0 + 16b + 0..15); lane l loads row l%16, K 8*(l/16)..+7 of the step (rows past T repeat
    // the last token)
    const bf16_t* asrc[LA];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int tok = min(t0 + 16 * (wave * LA + i) + lane % 16, T - 1);
        asrc[i] = x + (size_t)tok * d + (size_t)ks0 * 32 + 8 * (lane / 16);
    }
    // router block q = wave*LB + i (plane q / NB, column block q % NB); slots past NBL repeat
    // the last block, so every wave issues the same number of loads
    const size_t plane_stride = (size_t)NB * KS * 64;
    const u32x4* bsrc[LB];
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int q = min(wave * LB + i, NBL - 1);
        bsrc[i] = planes + (q / NB) * plane_stride + ((size_t)(q % NB) * KS + ks0) * 64 + lane;
    }
    auto issue = [&](int st, int stage) __attribute__((always_inline)) {
        u32x4* dst = lds + (size_t)stage * STAGE * 64;
#pragma unroll
        for (int i = 0; i < LA; ++i) gate_dma16(asrc[i] + (size_t)st * 32, dst + (wave * LA + i) * 64);
#pragma unroll
        for (int i = 0; i < LB; ++i) gate_dma16(bsrc[i] + (size_t)st * 64, dst + (ABLK + wave * LB + i) * 64);
    };
    // the K loop and the output of one column half: blocks [JB, JB + JN)
    auto run = [&](auto jb, auto jn) __attribute__((always_inline)) {
        constexpr int JB = decltype(jb)::value, JN = decltype(jn)::value;
        f32x4 acc[TPW][JN > 0 ? JN : 1];
#pragma unroll
        for (int tb = 0; tb < TPW; ++tb)
#pragma unroll
            for (int j = 0; j < JN; ++j) acc[tb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s0 = 0; s0 < STAGES - 1; ++s0) issue(min(s0, nsteps - 1), s0);
        gate_wait_vm_lds<(STAGES - 2) * L>();
        asm volatile("s_barrier" ::: "memory");
        for (int st = 0; st < nsteps; ++st) {
            // refill the stage read in the previous step (every wave passed this step's barrier
            // after its reads); past the last step it re-loads the last step into a stage that
            // is never read, so the wait counts stay uniform
            issue(min(st + STAGES - 1, nsteps - 1), (st + STAGES - 1) % STAGES);
            if constexpr (JN > 0) {
                const u32x4* sa = lds + (size_t)(st % STAGES) * STAGE * 64;
                const u32x4* sb = sa + ABLK * 64;
                bf16x8 af[TPW];
#pragma unroll
                for (int tb = 0; tb < TPW; ++tb) af[tb] = __builtin_bit_cast(bf16x8, sa[(tg * TPW + tb) * 64 + lane]);
#pragma unroll
                for (int pl = 2; pl >= 0; --pl) {  // smallest plane first
                    bf16x8 bf[JN];
#pragma unroll
                    for (int j = 0; j < JN; ++j) bf[j] = __builtin_bit_cast(bf16x8, sb[(pl * NB + JB + j) * 64 + lane]);
#pragma unroll
                    for (int tb = 0; tb < TPW; ++tb)
#pragma unroll
                        for (int j = 0; j < JN; ++j)
                            acc[tb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[tb], bf[j], acc[tb][j], 0, 0, 0);
                }
            }
            gate_wait_vm_lds<(STAGES - 2) * L>();  // step st+1 has landed (this wave's loads)
            asm volatile("s_barrier" ::: "memory");  // ... for every wave; stage st is free
        }
        gate_wait_vm_lds<0>();  // no LDS-DMA write may outlive the workgroup
        // lane holds column 16*j + lane%16, tokens 4*(lane/16) + i of each block
        float* out = part + ((size_t)blockIdx.y * T) * NC;
#pragma unroll
        for (int tb = 0; tb < TPW; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + 16 * (tg * TPW + tb) + 4 * (lane / 16) + i;
                if (t < T)
#pragma unroll
                    for (int j = 0; j < JN; ++j) out[(size_t)t * NC + 16 * (JB + j) + lane % 16] = acc[tb][j][i];
            }
    };
    if (ch == 0) run(std::integral_constant<int, 0>{}, std::integral_constant<int, NB0>{});
    else run(std::integral_constant<int, NB0>{}, std::integral_constant<int, NB - NB0>{});
}

// One wave per token: logits = the slices' partial sums added in slice order, + bias.
__global__ __launch_bounds__(256) void gate_mfma_finish(const float* __restrict__ part, int S, int NC, int T, int E,
                                                       int Ec, const float* __restrict__ bias, int k, int gflags,
                                                       int32_t* __restrict__ idx, float* __restrict__ w,
                                                       float* __restrict__ gs) {
    __shared__ float logits[4][kMaxExperts + 16];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int t = blockIdx.x * 4 + wave;
    if (t < T) {
        for (int c = lane; c < Ec; c += kWave) {
            // eight slices' loads in flight at a time, added in slice order
            const float* p = part + (size_t)t * NC + c;
            float v = 0.0f;
            for (int s0 = 0; s0 < S; s0 += 8) {
                float u[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) u[i] = s0 + i < S ? p[(size_t)(s0 + i) * T * NC] : 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) v += u[i];
            }
            logits[wave][c] = v + ((bias && c < E) ? bias[c] : 0.0f);
        }
    }
    __syncthreads();
    if (t < T) wave_topk_write(logits[wave], E, k, gflags, t, idx, w, gs);
}

// ---------------------------------------------------------------- prefill path, fp32 tokens
// 64 tokens x (16*EJ) router columns per workgroup; thread (ty, tx) owns tokens
// 4*ty..4*ty+3 and columns tx + 16*j. K advances in chunks of 32 with the next
// chunk held in registers while the current one is consumed from LDS.
constexpr int kTB = 64;
constexpr int kKC = 32;

template <typename XT, int EJ>
__global__ __launch_bounds__(256) void gate_tiled(const XT* __restrict__ x, const float* __restrict__ wr_t,
                                                  const float* __restrict__ bias, int T, int d, int E, int Ec,
                                                  int k, int gflags, int32_t* __restrict__ idx,
                                                  float* __restrict__ w, float* __restrict__ gs) {
    constexpr int ECP = 16 * EJ;
    constexpr int XP = kTB + 4;                       // padded token stride of the x tile
    constexpr int LP = ECP + 1;                       // padded stride of the logit tile
    constexpr int XS = 2 * kKC * XP;
    constexpr int WS = 2 * kKC * ECP;
    constexpr int SMEM = (XS + WS) > (kTB * LP) ? (XS + WS) : (kTB * LP);
    __shared__ float smem[SMEM];
    float* xs = smem;            // [2][KC][XP]   xs[k][token]
    float* ws = smem + XS;       // [2][KC][ECP]  ws[k][col]

    const int tid = threadIdx.x;
    const int ty = tid / 16, tx = tid % 16;
    const int t0 = blockIdx.x * kTB;

    // x chunk: thread loads 8 consecutive k of token tid/4 (64 tokens x 32 k)
    const int xl_tok = tid / 4, xl_k = (tid % 4) * 8;
    const bool xl_ok = t0 + xl_tok < T;
    const XT* xl_ptr = x + (size_t)(t0 + (xl_ok ? xl_tok : 0)) * d + xl_k;
    // w chunk: ECP rows x 32 k = ECP*8 float4; thread handles float4 q = tid + 256*i
    constexpr int WQ = (ECP * 8 + 255) / 256;

    float xr[8];
    float4 wr[WQ];
    auto gload = [&](int kc) {
        if (xl_ok) load8<XT>(xl_ptr + kc, xr);
        else {
#pragma unroll
            for (int v = 0; v < 8; ++v) xr[v] = 0.0f;
        }
#pragma unroll
        for (int i = 0; i < WQ; ++i) {
            int q = tid + 256 * i;
            int row = q / 8, c4 = q % 8;
            if (q < ECP * 8 && row < Ec)
                wr[i] = *reinterpret_cast<const float4*>(wr_t + (size_t)row * d + kc + c4 * 4);
            else
                wr[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto sstore = [&](int buf) {
        float* xb = xs + buf * kKC * XP;
        float* wb = ws + buf * kKC * ECP;
#pragma unroll
        for (int v = 0; v < 8; ++v) xb[(xl_k + v) * XP + xl_tok] = xr[v];
#pragma unroll
        for (int i = 0; i < WQ; ++i) {
            int q = tid + 256 * i;
            int row = q / 8, c4 = q % 8;
            if (q < ECP * 8) {
                wb[(c4 * 4 + 0) * ECP + row] = wr[i].x;
                wb[(c4 * 4 + 1) * ECP + row] = wr[i].y;
                wb[(c4 * 4 + 2) * ECP + row] = wr[i].z;
                wb[(c4 * 4 + 3) * ECP + row] = wr[i].w;
            }
        }
    };

    float acc[4][EJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < EJ; ++j) acc[i][j] = 0.0f;

    const int nk = d / kKC;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * kKC);
        const float* xb = xs + buf * kKC * XP;
        const float* wb = ws + buf * kKC * ECP;
#pragma unroll 8
        for (int kk = 0; kk < kKC; ++kk) {
            float4 xv = *reinterpret_cast<const float4*>(xb + kk * XP + ty * 4);
            float wv[EJ];
#pragma unroll
            for (int j = 0; j < EJ; ++j) wv[j] = wb[kk * ECP + tx + 16 * j];
#pragma unroll
            for (int j = 0; j < EJ; ++j) {
                acc[0][j] = fmaf(xv.x, wv[j], acc[0][j]);
                acc[1][j] = fmaf(xv.y, wv[j], acc[1][j]);
                acc[2][j] = fmaf(xv.z, wv[j], acc[2][j]);
                acc[3][j] = fmaf(xv.w, wv[j], acc[3][j]);
            }
        }
        if (kt + 1 < nk) sstore(buf ^ 1);
        __syncthreads();
    }
    // logits tile [64][LP] (reuses the staging buffers; all reads finished above)
    float* lt = smem;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < EJ; ++j) {
            int col = tx + 16 * j;
            float b = (bias && col < E) ? bias[col] : 0.0f;
            lt[(ty * 4 + i) * LP + col] = acc[i][j] + b;
        }
    __syncthreads();
    const int wave = tid / kWave;
    for (int r = wave; r < kTB; r += 4) {
        if (t0 + r < T) wave_topk_write(lt + r * LP, E, k, gflags, t0 + r, idx, w, gs);
    }
}

// ---------------------------------------------------------------- tiny batches, fused
// Gate and Scatter in one workgroup of 16 waves for up to four tokens: thread tid owns
// the K chunk [8*tid, 8*tid + 8) (d <= 8192); the chunks of every token and of eight
// router columns are loaded at once (a decode step is a chain of memory latencies, so
// one round trip instead of two or three), each wave folds its 64 partial dots with a
// butterfly, the 16 wave partials are added in LDS in a fixed order, one wave per token
// takes the top-k, and the same workgroup then runs the scatter ([0539edu §2.2], the
// two stages back to back with no launch between them). All loads of one CU pass its
// one address unit, so threads past d and tokens past T load nothing; the top-k results
// stay in LDS until the scatter starts, when the other waves store them, so no wait of
// the scatter's wave covers a store.
template <typename XT>
struct SmallGate {
    static constexpr int T = 4;  // tokens (register budget at 1024 threads)
    static constexpr int EC = 16;                      // router columns (experts + shared gate)
    static constexpr int EG = 8;                       // columns per load round
};

// MT: token slots (1 for a single token, whose instantiation holds a quarter of the dot
// code: its instructions are fetched cold at every decode step)
template <typename XT, int MT>
__global__ __launch_bounds__(1024) void gate_scatter_small(const XT* __restrict__ x, const float* __restrict__ wr_t,
                                                           const float* __restrict__ bias, int T, int d, int E,
                                                           int Ec, int k, int gflags, int32_t* __restrict__ idx,
                                                           float* __restrict__ w, float* __restrict__ gs, int V,
                                                           int bm, ScatterOut o) {
    static_assert(MT == 1 || MT == SmallGate<XT>::T, "token slots");
    constexpr int EC = SmallGate<XT>::EC, EG = SmallGate<XT>::EG;
    constexpr int NW = 16;
    __shared__ float part[NW][MT * EC];
    __shared__ float logits[MT][EC + 1];
    __shared__ ScatterWaveSmem sm;
    __shared__ int32_t s_idx[MT * kMaxTopK];  // the top-k results, stored by the other waves
    __shared__ float s_w[MT * kMaxTopK];
    __shared__ float s_gs[MT];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const bool has = tid * 8 < d;
    const int kc = has ? tid * 8 : 0;
    constexpr int XQ = sizeof(XT) / 2;  // 16-byte chunks per 8 elements
    // the first column group's router chunks are requested before the token rows, so both
    // are in flight together (the token rows' unpacking is hoisted above the column loop)
    u32x4 wq[EG][2];
    auto load_w = [&](int e0) {
#pragma unroll
        for (int g = 0; g < EG; ++g) {
            wq[g][0] = wq[g][1] = u32x4{0u, 0u, 0u, 0u};
            if (has && e0 + g < Ec) {
                const u32x4* p = reinterpret_cast<const u32x4*>(wr_t + (size_t)(e0 + g) * d + kc);
                wq[g][0] = p[0];
                wq[g][1] = p[1];
            }
        }
    };
    load_w(0);
    u32x4 xq[MT][XQ];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
        for (int q = 0; q < XQ; ++q) xq[t][q] = u32x4{0u, 0u, 0u, 0u};
        if (has && t < T) {
            const u32x4* p = reinterpret_cast<const u32x4*>(x + (size_t)t * d + kc);
#pragma unroll
            for (int q = 0; q < XQ; ++q) xq[t][q] = p[q];
        }
    }
    for (int e0 = 0; e0 < Ec; e0 += EG) {
        if (e0 > 0) load_w(e0);
        // per token, RG dots at a time, each group folded with one transposed butterfly
        constexpr int RG = 4;  // register budget at 1024 threads
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (t < T) {
#pragma unroll
                for (int g0 = 0; g0 < EG; g0 += RG) {
                    float acc[RG];
#pragma unroll
                    for (int r = 0; r < RG; ++r) {
                        float a = 0.0f;
#pragma unroll
                        for (int v = 0; v < 8; ++v) {
                            float f;
                            if constexpr (XQ == 1) {
                                const uint32_t u = xq[t][0][v / 2];
                                f = __uint_as_float((v & 1) ? (u & 0xFFFF0000u) : (u << 16));
                            } else {
                                f = __uint_as_float(xq[t][v / 4][v % 4]);
                            }
                            a = fmaf(f, __uint_as_float(wq[g0 + r][v / 4][v % 4]), a);
                        }
                        acc[r] = has ? a : 0.0f;
                    }
                    const float sum = wave_sum_many<RG>(acc);  // lane l: column e0 + g0 + l / (64 / RG)
                    const int g = g0 + lane / (64 / RG);
                    if (lane % (64 / RG) == 0 && e0 + g < Ec) part[wave][t * EC + e0 + g] = sum;
                }
            }
        }
    }
    __syncthreads();
    if (tid < T * EC) {
        const int t = tid / EC, e = tid - (tid / EC) * EC;
        if (e < Ec) {
            float v = 0.0f;
#pragma unroll
            for (int q = 0; q < NW; ++q) v += part[q][tid];
            logits[t][e] = v + ((bias && e < E) ? bias[e] : 0.0f);
        }
    }
    __syncthreads();
    if (wave < T) wave_topk_write(logits[wave], E, k, gflags, wave, s_idx, s_w, s_gs);
    __syncthreads();
    if (wave == 0) {
        scatter_wave(s_idx, T, E, k, V, bm, o, sm);  // at most 4 x 16 assignments
    } else {
        const int i0 = tid - kWave, n = blockDim.x - kWave;
        for (int i = i0; i < T * k; i += n) {
            idx[i] = s_idx[i];
            w[i] = s_w[i];
        }
        if ((gflags & kGateShared) && i0 < T) gs[i0] = s_gs[i0];
    }
}

// ---------------------------------------------------------------- decode batches, split
// For T <= 64 the router GEMM is spread over many workgroups, each one 16-column block
// times one 128-wide K slice for every token (a decode step is a chain of memory
// latencies: every load of a workgroup is issued at once, and many CUs pull the router):
//   gate_partial: lane (column e = lane%16, 32-wide sub-slice c = lane/16) keeps its 32
//     router weights in registers; wave w (of 16) takes tokens w, w+16, w+32, w+48, all
//     their loads first; one fp32 dot per token, the four sub-slices folded with two
//     butterflies, written to part[slice][t][column];
//   gate_finish: one workgroup adds the slices in order (+ bias), takes the top-k of every
//     token and then runs the scatter, so the routing is done in two launches.
constexpr int kPartK = 128;  // K slice per gate_partial workgroup

template <typename XT>
__global__ __launch_bounds__(1024) void gate_partial(const XT* __restrict__ x, const float* __restrict__ wr_t, int T,
                                                     int d, int Ec, float* __restrict__ part) {
    constexpr int XQ = sizeof(XT) / 2;   // 16-byte chunks per 8 elements
    constexpr int U = XQ == 1 ? 4 : 2;   // tokens per wave per round (register budget)
    const int nb = blockIdx.x, ks = blockIdx.y, NC = gridDim.x * 16;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int e = nb * 16 + lane % 16;
    const int k0 = ks * kPartK + (lane / 16) * 32;
    const bool kin = k0 < d;  // d % 32 == 0: a sub-slice is all inside or all outside
    const int kc = kin ? k0 : 0;
    float wv[32];
    {
        const float4* p = reinterpret_cast<const float4*>(wr_t + (size_t)(e < Ec ? e : 0) * d + kc);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 q = p[i];
            wv[4 * i] = q.x;
            wv[4 * i + 1] = q.y;
            wv[4 * i + 2] = q.z;
            wv[4 * i + 3] = q.w;
        }
    }
    for (int t0 = wave; t0 < T; t0 += 16 * U) {
        u32x4 xq[U][4 * XQ];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = t0 + 16 * u;
            const u32x4* px = reinterpret_cast<const u32x4*>(x + (size_t)(t < T ? t : 0) * d + kc);
#pragma unroll
            for (int i = 0; i < 4 * XQ; ++i) xq[u][i] = px[i];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = t0 + 16 * u;
            float acc = 0.0f;
#pragma unroll
            for (int v = 0; v < 32; ++v) {
                float f;
                if constexpr (XQ == 1) {
                    const uint32_t q = xq[u][v / 8][(v % 8) / 2];
                    f = __uint_as_float((v & 1) ? (q & 0xFFFF0000u) : (q << 16));
                } else {
                    f = __uint_as_float(xq[u][v / 4][v % 4]);
                }
                acc = fmaf(f, wv[v], acc);
            }
            acc = kin ? acc : 0.0f;
            acc += __shfl_xor(acc, 16, kWave);
            acc += __shfl_xor(acc, 32, kWave);
            if (lane < 16 && t < T) part[((size_t)ks * T + t) * NC + e] = acc;
        }
    }
}

constexpr int kFinishT = 64;  // tokens per gate_finish (the decode bound)

__global__ __launch_bounds__(1024) void gate_finish(const float* __restrict__ part, int KS, int NC, int T, int E,
                                                    int Ec, const float* __restrict__ bias, int k, int gflags,
                                                    int32_t* __restrict__ idx, float* __restrict__ w,
                                                    float* __restrict__ gs, int V, int bm, ScatterOut o) {
    constexpr int NW = 16;
    __shared__ float logits[kFinishT][kMaxExperts + 2];
    __shared__ int32_t ids[kFinishT * 8];  // top-k ids (k <= 8 here) for the scatter to read from LDS
    __shared__ ScatterWaveSmem sm;
    __shared__ ScatterSmem<NW> smb;
    const int tid = threadIdx.x, wave = tid / kWave;
    for (int i = tid; i < T * Ec; i += NW * kWave) {
        const int t = i / Ec, e = i - (i / Ec) * Ec;
        // slices added in order; their loads are issued 16 at a time (not one round trip each)
        float v = 0.0f;
        for (int q0 = 0; q0 < KS; q0 += 16) {
            float pv[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) pv[q] = q0 + q < KS ? part[((size_t)(q0 + q) * T + t) * NC + e] : 0.0f;
#pragma unroll
            for (int q = 0; q < 16; ++q) v += pv[q];
        }
        logits[t][e] = v + ((bias && e < E) ? bias[e] : 0.0f);
    }
    __syncthreads();
    for (int t = wave; t < T; t += NW) wave_topk_write(logits[t], E, k, gflags, t, idx, w, gs, ids);
    __syncthreads();
    if (T * k <= kScatterWaveMaxN) {
        if (wave == 0) scatter_wave(ids, T, E, k, V, bm, o, sm);
    } else {
        scatter_block<NW>(ids, T, E, k, V, bm, o, smb);
    }
}

template <int NB>
hipError_t launch_gate_mfma_nb(const bf16_t* x, const u32x4* planes, const float* bias, int T, int d, int E,
                               int k, int gflags, int32_t* idx, float* w, float* gs, float* part, size_t part_cap,
                               hipStream_t s) {
    constexpr int LB = (3 * NB + 7) / 8;  // as in the kernel (8 waves)
    constexpr size_t lds_bytes = (size_t)kGateStages * (4 * kGateTPW + 8 * LB) * 1024;
    static_assert(lds_bytes <= 160 * 1024, "LDS");
    auto kern = gate_mfma_part<NB>;
    static bool attr_set = false;  // one-time opt-in above the default dynamic LDS limit
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)lds_bytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int S = gate_mfma_slices(T, d), kps = gate_mfma_kps(T, d);
    if (d % 32 || (S - 1) * kps >= d / 32) return hipErrorInvalidValue;
    if ((size_t)S * T * NB * 16 * sizeof(float) > part_cap) return hipErrorInvalidValue;  // partial logits fit
    hipLaunchKernelGGL(kern, dim3(gate_mfma_tiles(T), S), dim3(512), lds_bytes, s, x, planes, T, d, kps, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const bool has_shared = (gflags & kGateShared) != 0;
    hipLaunchKernelGGL(gate_mfma_finish, dim3((T + 3) / 4), dim3(256), 0, s, (const float*)part, S, NB * 16, T, E,
                       E + (has_shared ? 1 : 0), bias, k, gflags, idx, w, gs);
    return hipGetLastError();
}

hipError_t launch_gate_mfma(int NB, const bf16_t* x, const u32x4* planes, const float* bias, int T, int d, int E,
                            int k, int gflags, int32_t* idx, float* w, float* gs, float* part, size_t part_cap,
                            hipStream_t s) {
    switch (NB) {
#define GATE_MFMA_CASE(J) \
    case J: return launch_gate_mfma_nb<J>(x, planes, bias, T, d, E, k, gflags, idx, w, gs, part, part_cap, s);
        GATE_MFMA_CASE(1) GATE_MFMA_CASE(2) GATE_MFMA_CASE(3) GATE_MFMA_CASE(4) GATE_MFMA_CASE(5)
        GATE_MFMA_CASE(6) GATE_MFMA_CASE(7) GATE_MFMA_CASE(8) GATE_MFMA_CASE(9)
#undef GATE_MFMA_CASE
        default: return hipErrorInvalidValue;
    }
}

// per-token dots for decode batches, but routers wider than 16 columns with bf16 tokens
// past kGateSplitMaxT tokens, which the MFMA path serves faster
bool use_rowdot(int T, int d, int Ec, bool has_planes) {
    return T <= 64 && d <= 2048 * kRowXC && (Ec <= 16 || !has_planes || T <= kGateSplitMaxT);
}

template <typename XT>
hipError_t launch_gate_t(const XT* x, const float* wr_t, const u32x4* planes, const float* bias, int T, int d, int E,
                         int gflags, int k, int32_t* idx, float* w, float* gs, float* part, size_t part_cap,
                         hipStream_t s) {
    const bool has_shared = (gflags & kGateShared) != 0;
    const int Ec = E + (has_shared ? 1 : 0);
    if (use_rowdot(T, d, Ec, planes != nullptr)) {
        switch ((d + 2047) / 2048) {
#define ROWDOT_CASE(C)                                                                                            \
    case C:                                                                                                       \
        hipLaunchKernelGGL((gate_rowdot<XT, C>), dim3(T), dim3(256), 0, s, x, wr_t, bias, d, E, Ec, k, gflags, idx, \
                           w, gs);                                                                                \
        break;
            ROWDOT_CASE(1) ROWDOT_CASE(2) ROWDOT_CASE(3) ROWDOT_CASE(4)
#undef ROWDOT_CASE
            default:
                return hipErrorInvalidValue;
        }
    } else if (planes != nullptr) {
        if (part == nullptr) return hipErrorInvalidValue;
        return launch_gate_mfma((Ec + 15) / 16, (const bf16_t*)x, planes, bias, T, d, E, k, gflags, idx, w, gs, part,
                                part_cap, s);
    } else {
        const int EJ = (Ec + 15) / 16;
        dim3 grid((T + kTB - 1) / kTB);
        switch (EJ) {
#define GATE_CASE(J)                                                                                          \
    case J:                                                                                                   \
        hipLaunchKernelGGL((gate_tiled<XT, J>), grid, dim3(256), 0, s, x, wr_t, bias, T, d, E, Ec, k,         \
                           gflags, idx, w, gs);                                                               \
        break;
            GATE_CASE(1) GATE_CASE(2) GATE_CASE(3) GATE_CASE(4) GATE_CASE(5)
            GATE_CASE(6) GATE_CASE(7) GATE_CASE(8) GATE_CASE(9)
#undef GATE_CASE
            default:
                return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

}  // namespace

bool gate_split_fits(int T, int k) { return T >= 1 && T <= kFinishT && k <= 8; }

size_t gate_split_workspace(int T, int d, int E, bool has_shared) {
    const int NC = (E + (has_shared ? 1 : 0) + 15) / 16 * 16;
    return (size_t)((d + kPartK - 1) / kPartK) * T * NC * sizeof(float);
}

hipError_t launch_gate_split(const void* x, bool x_bf16, const float* wr_t, const float* bias, int T, int d, int E,
                             int gflags, int k, int32_t* idx, float* w, float* gs, int V, int bm,
                             const ScatterOut& o, float* part, hipStream_t s) {
    const bool has_shared = (gflags & kGateShared) != 0;
    if (!gate_split_fits(T, k) || d % 32 || E > kMaxExperts || E + V > kMaxEt) return hipErrorInvalidValue;
    const int Ec = E + (has_shared ? 1 : 0);
    const int NB = (Ec + 15) / 16, KS = (d + kPartK - 1) / kPartK;
    if (x_bf16)
        hipLaunchKernelGGL(gate_partial<bf16_t>, dim3(NB, KS), dim3(1024), 0, s, (const bf16_t*)x, wr_t, T, d, Ec,
                           part);
    else
        hipLaunchKernelGGL(gate_partial<float>, dim3(NB, KS), dim3(1024), 0, s, (const float*)x, wr_t, T, d, Ec,
                           part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gate_finish, dim3(1), dim3(1024), 0, s, (const float*)part, KS, NB * 16, T, E, Ec, bias, k,
                       gflags, idx, w, gs, V, bm, o);
    return hipGetLastError();
}

bool gate_scatter_small_fits(int T, int d, int E, bool has_shared, bool x_bf16) {
    const int mt = x_bf16 ? SmallGate<bf16_t>::T : SmallGate<float>::T;
    return T >= 1 && T <= mt && d <= 8 * 1024 && d % 8 == 0 && E + (has_shared ? 1 : 0) <= SmallGate<float>::EC;
}

hipError_t launch_gate_scatter_small(const void* x, bool x_bf16, const float* wr_t, const float* bias, int T, int d,
                                     int E, int gflags, int k, int32_t* idx, float* w, float* gs, int V,
                                     int bm, const ScatterOut& o, hipStream_t s) {
    const bool has_shared = (gflags & kGateShared) != 0;
    if (!gate_scatter_small_fits(T, d, E, has_shared, x_bf16) || E + V > kMaxEt) return hipErrorInvalidValue;
    const int Ec = E + (has_shared ? 1 : 0);
    if (x_bf16) {
        auto kern = T == 1 ? gate_scatter_small<bf16_t, 1> : gate_scatter_small<bf16_t, SmallGate<bf16_t>::T>;
        hipLaunchKernelGGL(kern, dim3(1), dim3(1024), 0, s, (const bf16_t*)x, wr_t, bias, T, d, E, Ec, k, gflags,
                           idx, w, gs, V, bm, o);
    } else {
        auto kern = T == 1 ? gate_scatter_small<float, 1> : gate_scatter_small<float, SmallGate<float>::T>;
        hipLaunchKernelGGL(kern, dim3(1), dim3(1024), 0, s, (const float*)x, wr_t, bias, T, d, E, Ec, k, gflags, idx,
                           w, gs, V, bm, o);
    }
    return hipGetLastError();
}

size_t gate_mfma_workspace(int T, int d, int E, bool has_shared, bool x_bf16) {
    const int Ec = E + (has_shared ? 1 : 0);
    if (T <= 0 || !x_bf16 || use_rowdot(T, d, Ec, true)) return 0;
    return (size_t)gate_mfma_slices(T, d) * T * ((Ec + 15) / 16 * 16) * sizeof(float);
}

size_t gate_mfma_workspace_max(int Tmax, int E, bool has_shared) {
    // slices <= ceil(256 / tiles) <= 256 / tiles + 1 and T <= tiles * (tokens per tile), so
    // slices * T <= 256 * (tokens per tile) + T
    const int Ec = E + (has_shared ? 1 : 0);
    return ((size_t)256 * 64 * kGateTPW + (size_t)Tmax) * ((Ec + 15) / 16 * 16) * sizeof(float);
}

hipError_t launch_gate(const void* x, bool x_bf16, const float* wr_t, const void* planes, const float* bias, int T,
                       int d, int E, int gflags, int k, int32_t* idx, float* w, float* gs, float* part,
                       size_t part_cap, hipStream_t s) {
    if (x_bf16)
        return launch_gate_t<bf16_t>((const bf16_t*)x, wr_t, (const u32x4*)planes, bias, T, d, E, gflags, k, idx, w,
                                     gs, part, part_cap, s);
    return launch_gate_t<float>((const float*)x, wr_t, nullptr, bias, T, d, E, gflags, k, idx, w, gs, nullptr, 0, s);
}

}  // namespace moe
