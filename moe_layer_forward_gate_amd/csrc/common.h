// Internal declarations shared by the libmoe HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // bfloat16 bit pattern
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16-byte chunk (a native vector, so copies stay in registers)

constexpr int kWave = 64;
constexpr int kMaxExperts = 128;   // routed experts
constexpr int kMaxTopK = 64;       // one wave lane per slot in the weight softmax
constexpr int kXcds = 8;           // MI355X: workgroups are dealt round-robin to 8 XCDs

// bf16 <-> fp32. Widening is exact; narrowing rounds to nearest, ties to even,
// by integer rounding of the fp32 bit pattern (inputs are finite).
__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// ------------------------------------------------------------------ launchers
// Gate flags: kGateShared -- router column E is the shared expert's gate (its sigmoid
// goes to gs); kGateClamp -- the routed logits are clamped to [-kGateClampAbs,
// kGateClampAbs] before the top-k and the softmax; kGateRaw -- the routing weights are
// the chosen (clamped, when kGateClamp) logits themselves instead of their softmax.
constexpr int kGateShared = 1, kGateClamp = 2, kGateRaw = 4;
constexpr float kGateClampAbs = 50.0f;
// Gate: router logits, top-k with (logit desc, id asc) order, softmax weights over
// the chosen logits, and (with kGateShared) the shared-expert sigmoid gate read
// from router column E. wr_t is the router weight transposed to [Ec][d].
// planes: the router weight split into three bf16 planes in fragment order (bf16 tokens only).
// part: at least gate_mfma_workspace(T, d, E, has_shared, x_bf16) bytes (part_cap: its size,
// checked before the launch) for the partial logits of the MFMA gate (bf16 tokens past the
// per-token decode gate), else unused. gate_mfma_workspace_max bounds that over T <= Tmax.
hipError_t launch_gate(const void* x, bool x_bf16, const float* wr_t, const void* planes, const float* bias, int T,
                       int d, int E, int gflags, int k, int32_t* idx, float* w, float* gs, float* part,
                       size_t part_cap, hipStream_t s);
size_t gate_mfma_workspace(int T, int d, int E, bool has_shared, bool x_bf16);
size_t gate_mfma_workspace_max(int Tmax, int E, bool has_shared);

// Scatter: counts, offsets and the stable by-expert permutation of the T*k routed
// assignments, V shared virtual experts appended (each takes every token), and the
// per-expert tile starts for row tiles of height bm.
struct ScatterOut {
    int32_t* counts;        // [Et]
    int32_t* offsets;       // [Et+1]
    int32_t* tile_start;    // [Et+1]
    int32_t* sorted_c;      // [P]: combine slot c = t*kt + j of each sorted row
    int32_t* user_counts;   // [E] or null
    int32_t* user_offsets;  // [E+1] or null
    int32_t* user_sorted;   // [T*k] or null: a = t*k + j
};
hipError_t launch_scatter(const int32_t* idx, int T, int E, int k, int V, int bm, const ScatterOut& o,
                          hipStream_t s);
// The same scatter over many workgroups (three launches), for large T*k; `work` holds
// scatter_wide_workspace(T*k, E) bytes.
size_t scatter_wide_workspace(int N, int E);
hipError_t launch_scatter_wide(const int32_t* idx, int T, int E, int k, int V, int bm, const ScatterOut& o,
                               int32_t* work, hipStream_t s);
// Gate then Scatter for decode batches (T <= 64, k <= 8) in two launches: partial router
// dots over (16-column block, 128-wide K slice) workgroups into `part`
// (gate_split_workspace bytes), then one workgroup for the sums, top-k and scatter.
bool gate_split_fits(int T, int k);
// Routers wider than 16 columns with bf16 tokens take the split gate (or the per-token
// one) up to this batch and the MFMA gate past it: the split gate's one-workgroup finish
// grows with T (64-expert + shared layer, T = 64: 50 us split, 30 us MFMA; T = 16: 24 us
// split, 30 us MFMA).
constexpr int kGateSplitMaxT = 24;
size_t gate_split_workspace(int T, int d, int E, bool has_shared);
hipError_t launch_gate_split(const void* x, bool x_bf16, const float* wr_t, const float* bias, int T, int d, int E,
                             int gflags, int k, int32_t* idx, float* w, float* gs, int V, int bm,
                             const ScatterOut& o, float* part, hipStream_t s);
// Gate then Scatter in a single workgroup, for tiny batches: up to 4 tokens,
// d_model <= 8192, at most 16 router columns (experts + shared gate).
bool gate_scatter_small_fits(int T, int d, int E, bool has_shared, bool x_bf16);
hipError_t launch_gate_scatter_small(const void* x, bool x_bf16, const float* wr_t, const float* bias, int T, int d,
                                     int E, int gflags, int k, int32_t* idx, float* w, float* gs, int V,
                                     int bm, const ScatterOut& o, hipStream_t s);

// Grouped expert GEMMs on bf16 MFMA (expert weights bf16 or int8 in fragment order).
struct GemmArgs {
    const int32_t* tile_start;  // [Et+1]
    const int32_t* offsets;     // [Et+1]
    const int32_t* sorted_c;    // [P]
    int Et, kt, k;              // experts incl. virtual, slots per token incl. virtual, routed k
    int max_tiles;              // bound on sum_e ceil(n_e / bm)
    int bm;                     // row tile height: tiled 256 (bf16), 128 (int8), 64 (int4); streaming 16-64;
                                // must match the scatter's tile list
    int ksplit;                 // down projection: K split into ksplit partial sums (ow rows c*ksplit + s)
    int merge_shared;           // tiled down projection: shared slices summed as one K = V*F tile (ksplit 1)
    int weights_once;           // streaming kernels: an expert's weights are read by one row tile only
                                // (non-temporal loads), else by several (cached loads: re-reads hit)
    // Streaming kernels: A = x rows gathered by token (up), H rows [P][F] (down).
    // Tiled kernels: A in fragment order over padded rows (tile g owns padded rows
    // [g*bm, (g+1)*bm)): xp = the gathered tokens [R/16][d/32][64][8] written by
    // launch_pack_a, h = H as [R/16][F/32][64][8] written by the up kernel.
    const bf16_t* x;            // [T][d]
    bf16_t* xp;                 // tiled up operand (see above)
    bf16_t* h;                  // [P][F] or packed [R/16][F/32][64][8]
    const void* wgu;            // packed gate/up
    const void* wdn;            // packed down
    const float* s_gate;        // int8: [E][F]; int4: the up projection's [E][d/128][2F] (packed column order)
    const float* s_up;          // int8: [E][F]
    const float* s_down;        // int8: [E][d]; int4: [E][F/128][d]
    const float* topk_w;        // [T][k]
    const float* gs;            // [T] shared gate or null
    float* ow;                  // [T*kt*ksplit][d] weighted expert outputs (partial sums)
    int d, F;
    int T;                      // tokens of the batch (a tile holds at most min(bm, T * k) rows)
    // The down projection's row tiling, which H follows: tile table [Et+1] and height (a
    // multiple of 16). The same as tile_start / bm but for the int4 tile-stream GEMMs at
    // 41-72 rows per expert, whose up projection takes 80-row tiles (an expert's weights
    // streamed once) and down projection 64-row ones; launch_pack_a then fills
    // tile_start_h from the offsets.
    int32_t* tile_start_h;
    int bm_h;
};
// LDS-tiled MFMA GEMMs; wq: the weight kind (kWBf16, kWI8, kWI4), with a.bm 256, 128, 64
hipError_t launch_expert_up_tiled(const GemmArgs& a, int wq, hipStream_t s);
hipError_t launch_expert_down_tiled(const GemmArgs& a, int wq, hipStream_t s);
// The same GEMMs with the weights streamed into registers and the row tile staged in LDS
// (a.bm 128 or 160 for bf16, 64 or 128 for int8, 64 for int4 and 80 for its up projection;
// N % 256 == 0)
hipError_t launch_expert_up_tstream(const GemmArgs& a, int wq, hipStream_t s);
hipError_t launch_expert_down_tstream(const GemmArgs& a, int wq, hipStream_t s);
// The int8 tile-stream down projection takes two column blocks per wave (128 columns per
// workgroup) while the experts average at most 64 rows (T * k routed rows over E experts).
inline bool tstream_narrow_down(int T, int k, int E) { return (long long)T * k <= 64LL * E; }
// Token rows into the tiled up operand a.xp (padded rows past an expert's last row are
// zero; shared virtual experts after the first are not written, the up kernel reads the
// first one's rows for them). Reads the scatter's tile list on the device; writes
// max_tiles*bm rows at most.
hipError_t launch_pack_a(const GemmArgs& a, hipStream_t s);
// A caller's routing (ids [N], weights [N]) into the layer's buffers: ids outside
// [0, E) become expert 0 with weight 0.
hipError_t launch_route_in(const int32_t* idx, const float* w, int N, int E, int32_t* idx_out, float* w_out,
                           hipStream_t s);
// Small-batch variants (a.bm = 16, 32 or 64: an active expert usually fits one row tile;
// one that does not takes several, each streaming the weights again).
// wq: the weight kind, kWBf16, kWI8 (per-channel scales s_gate/s_up/s_down) or kWI4
// (group scales: s_gate = the up projection's [E][d/128][2F] in packed column order,
// s_down = [E][F/128][d]).
constexpr int kWBf16 = 0, kWI8 = 1, kWI4 = 2;
hipError_t launch_expert_up_stream(const GemmArgs& a, int wq, hipStream_t s);
hipError_t launch_expert_down_stream(const GemmArgs& a, int wq, hipStream_t s);
constexpr int kStreamMaxT = 64;     // largest T served by the streaming kernels
constexpr int kStreamMaxSplit = 16; // largest K split of their down projection

// fp32 experts (VALU), weights in natural [E][K][N] layout.
struct GemmF32Args {
    const int32_t* tile_start;
    const int32_t* offsets;
    const int32_t* sorted_c;
    int Et, kt, k, max_tiles;
    const float* x;      // [T][d]
    float* h;            // [P][F]
    const float* wg;     // [E][d][F]
    const float* wu;     // [E][d][F]
    const float* wd;     // [E][F][d]
    const float* topk_w;
    const float* gs;
    float* ow;
    int d, F;
};
hipError_t launch_expert_up_f32(const GemmF32Args& a, hipStream_t s);
hipError_t launch_expert_down_f32(const GemmF32Args& a, hipStream_t s);

// Gather: y[t] = sum_{j < nrow} ow[t*stride + j], written as bf16 or fp32 (rows: slots x K
// splits; stride >= nrow rows per token).
hipError_t launch_combine(const float* ow, int T, int nrow, int stride, int d, void* y, bool y_bf16,
                          hipStream_t s);

// Create-time repacking into fragment order (see pack.hip).
hipError_t pack_router(const float* wr, const float* ws_gate_vec, int d, int E, float* wr_t, hipStream_t s);
// Router weight [d][E] (+ shared gate column E) as three bf16 planes hi + mid + lo in MFMA
// B-fragment order: [3][NB = ceil(Ec/16)][d/32][64 lanes][8], columns past Ec zero.
hipError_t pack_router_planes(const float* wr, const float* ws_gate_vec, int d, int E, bf16_t* planes,
                              hipStream_t s);
hipError_t pack_gu_bf16(const bf16_t* wg, const bf16_t* wu, int E, int d, int F, bf16_t* dst,
                        int64_t src_ld, hipStream_t s);
hipError_t pack_dn_bf16(const bf16_t* wd, int E, int F, int d, bf16_t* dst, hipStream_t s);
hipError_t pack_gu_i8(const int8_t* wg, const int8_t* wu, int E, int d, int F, int8_t* dst, hipStream_t s);
hipError_t pack_dn_i8(const int8_t* wd, int E, int F, int d, int8_t* dst, hipStream_t s);
// int4 (two per byte along K, low nibble first, two's complement) into 1 KB blocks of
// 16 columns x 128 K (one scale group): lane l's four words hold column l%16, K rows
// 32*s + 8*(l/16) + 0..7 of word s as codes q + 8, rows 2i in nibble i and 2i+1 in
// nibble i+4; and the group scales [E][K/128][N] into the packed column order.
hipError_t pack_gu_i4(const uint8_t* wg, const uint8_t* wu, int E, int d, int F, uint8_t* dst, hipStream_t s);
hipError_t pack_dn_i4(const uint8_t* wd, int E, int F, int d, uint8_t* dst, hipStream_t s);
hipError_t pack_scales_gu_i4(const float* sg, const float* su, int E, int d, int F, float* dst, hipStream_t s);

// Row tile height of the fp32 GEMMs (the bf16/int8 GEMMs take 256 or 128, chosen per call).
constexpr int kBMf32 = 64;
constexpr int kMaxVirtual = 63;  // shared-expert slices (scatter scan limit)

// One output tile of a grouped expert GEMM: expert e, rows [seg0 + row0, seg0 +
// row0 + rows) of the by-expert order, column tile n; g = tile_start[e] + row0/bm is
// the tile's index in the padded row space of the tiled operands.
struct Tile {
    int e, row0, rows, seg0, n, g;
};

// Map this workgroup to a tile. Tiles are ordered expert by expert; inside an
// expert, column tiles come in groups of GN, and within a group the GN column tiles
// of a row tile run together, row tile after row tile, so workgroups that share a
// weight tile (same n) or an activation tile (same row0) run close together.
// Workgroup i is dealt to XCD i % 8 by the hardware; the logical index is remapped
// so each XCD works on contiguous tiles and keeps their weight/activation tiles in
// its own L2: one stretch of total/8 tiles per XCD (chunk = 0), or chunks of `chunk`
// consecutive tiles dealt to the XCDs in turn, which spreads the cheap ragged tiles
// of the experts' last rows, and any run of costlier tiles, over all XCDs.
// tile_start[e] = sum of ceil(n_e' / bm) over e' < e; it and offsets are read
// from device memory (the scatter just wrote them), so the grid is launched for
// an upper bound and idle workgroups return at once.
__device__ __forceinline__ bool decode_tile_at(const int32_t* __restrict__ ts, const int32_t* __restrict__ offs,
                                               int Ecount, int NT, int GN, int bm, int S, int i, Tile& tl,
                                               int& split, int chunk = 0) {
    // i: the workgroup's index in the launch, dealt to XCD i % 8; S K-splits of every tile
    // (logical index = tile * S + split), the XCD remap applied to the combined index
    const int NTp = (NT + GN - 1) / GN * GN;
    const int total = ts[Ecount] * NTp * S;
    const int slot = i / kXcds, xcd = i % kXcds;
    int L;
    if (chunk > 0) {
        // the launch holds at least total + kXcds * chunk workgroups
        const int per = (total + kXcds * chunk - 1) / (kXcds * chunk) * chunk;
        if (slot >= per) return false;
        L = ((slot / chunk) * kXcds + xcd) * chunk + slot % chunk;
    } else {
        const int per = (total + kXcds - 1) / kXcds;
        if (slot >= per) return false;
        L = xcd * per + slot;
    }
    if (L >= total) return false;
    const int Lt = L / S;
    split = L - Lt * S;
    const int lane = threadIdx.x % kWave;
    int c = 0;
    for (int j0 = 0; j0 <= Ecount; j0 += kWave) {
        const int j = j0 + lane;
        const bool ok = j <= Ecount && ts[j] * NTp <= Lt;
        c += __popcll(__ballot(ok));
    }
    const int e = c - 1;
    const int t0 = ts[e], mt = ts[e + 1] - t0;
    const int local = Lt - t0 * NTp;
    const int grp = local / (mt * GN);
    const int rem = local - grp * mt * GN;
    const int m = rem / GN;
    const int n = grp * GN + (rem - m * GN);
    if (n >= NT) return false;
    tl.e = e;
    tl.n = n;
    tl.g = t0 + m;
    tl.row0 = m * bm;
    tl.seg0 = offs[e];
    tl.rows = min(bm, offs[e + 1] - tl.seg0 - tl.row0);
    return true;
}

__device__ __forceinline__ bool decode_tile(const int32_t* __restrict__ ts, const int32_t* __restrict__ offs,
                                            int Et, int NT, int GN, int bm, Tile& tl) {
    int split;
    return decode_tile_at(ts, offs, Et, NT, GN, bm, 1, blockIdx.x, tl, split);
}

// decode_tile over S K-splits of every tile.
__device__ __forceinline__ bool decode_tile_split(const int32_t* __restrict__ ts, const int32_t* __restrict__ offs,
                                                  int Et, int NT, int GN, int bm, int S, Tile& tl, int& split,
                                                  int chunk = 0) {
    return decode_tile_at(ts, offs, Et, NT, GN, bm, S, blockIdx.x, tl, split, chunk);
}

// Down projection with the shared expert's V slices merged into one K = V*F sum per
// tile: workgroups 0 .. mtv*NT-1 take the row tiles of the first slice (expert E0, all
// slices hold the same rows), one per XCD in turn and launched first (each runs V times
// longer than a routed tile); the rest, from the next multiple of 8, take the routed
// experts' tiles through decode_tile_at. *kv = V for a merged tile, 1 otherwise.
__device__ __forceinline__ bool decode_tile_down_merged(const int32_t* __restrict__ ts,
                                                        const int32_t* __restrict__ offs, int E0, int V, int NT,
                                                        int GN, int bm, Tile& tl, int& kv) {
    const int mtv = ts[E0 + 1] - ts[E0];
    const int nlong = mtv * NT;
    const int i = blockIdx.x;
    if (i < nlong) {
        const int m = i / NT;
        tl.e = E0;
        tl.n = i - m * NT;
        tl.g = ts[E0] + m;
        tl.row0 = m * bm;
        tl.seg0 = offs[E0];
        tl.rows = min(bm, offs[E0 + 1] - tl.seg0 - tl.row0);
        kv = V;
        return true;
    }
    const int first = (nlong + kXcds - 1) / kXcds * kXcds;  // keeps i % 8 the XCD of the remap
    if (i < first) return false;
    int split;
    kv = 1;
    return decode_tile_at(ts, offs, E0, NT, GN, bm, 1, i - first, tl, split);
}

}  // namespace moe
