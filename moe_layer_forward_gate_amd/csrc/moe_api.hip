// libmoe C ABI: argument checks, layer creation (packing + workspace), the
// forward pass as a fixed sequence of launches on the caller's stream, and
// teardown. The host side plans launch shapes from T, k and the layer shape
// ([hotelren §2.2]: grid, block and shared memory come from the batch and top-k,
// computed by the host); everything that depends on the routing itself (expert
// counts, tile lists) stays on the device, so a forward never waits on the host.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <new>

#include "../../include/moe.h"
#include "common.h"

using namespace moe;

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

#define HIP_TRY(expr)                                                                                       \
    do {                                                                                                    \
        hipError_t e_ = (expr);                                                                             \
        if (e_ != hipSuccess) return fail(MOE_EHIP, "%s: %s (%s:%d)", #expr, hipGetErrorString(e_), __FILE__, \
                                          __LINE__);                                                        \
    } while (0)

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

// Per-call workspace of a forward: routing tables, the gathered GEMM operand, H and the
// combine rows. A layer owns one sized for desc.max_tokens; the allocation-free forward
// carves one out of the device's static scratch for the call's own T.
struct Work {
    int32_t* counts = nullptr;
    int32_t* offsets = nullptr;
    int32_t* tile_start = nullptr;
    int32_t* tile_start_h = nullptr;  // the down projection's tile table when its tiling differs
    int32_t* sorted_c = nullptr;
    float* gs = nullptr;
    int32_t* ridx = nullptr;  // a caller's routing, checked (moe_forward_routed)
    float* rw = nullptr;
    float* gate_part = nullptr;  // partial router dots of the split decode gate or the MFMA gate
    size_t gate_part_bytes = 0;
    int32_t* scatter_work = nullptr;  // chunk counts and ranks of the multi-workgroup scatter
    bf16_t* xp = nullptr;  // tiled up operand (bf16/int8 experts)
    void* h = nullptr;
    float* ow = nullptr;
};

struct moe_layer {
    moe_desc desc{};
    int device = 0;
    int cus = 256;  // compute units of the device
    int E = 0, V = 0, Et = 0, kt = 0, Ec = 0;
    bool has_bias = false;
    // packed weights
    float* wr_t = nullptr;
    bf16_t* wr_planes = nullptr;  // router as three bf16 planes (bf16 activations)
    float* bias = nullptr;
    void* wgu = nullptr;
    void* wdn = nullptr;
    float* s_gate = nullptr;
    float* s_up = nullptr;
    float* s_down = nullptr;
    // workspace for max_tokens
    Work w;
    size_t ow_rows = 0;  // combine rows of that workspace (bounds the plans' K splits)
    // profiling
    bool profiling = false;
    hipEvent_t ev[6] = {};
    bool ran = false;
};

namespace {

void release(moe_layer* L) {
    if (!L) return;
    const Work& w = L->w;
    void* bufs[] = {L->wr_t, L->wr_planes, L->bias, L->wgu, L->wdn, L->s_gate, L->s_up, L->s_down, w.counts, w.offsets,
                    w.tile_start, w.tile_start_h, w.sorted_c, w.gs, w.ridx, w.rw, w.gate_part, w.scatter_work,
                    w.xp, w.h, w.ow};
    for (void* p : bufs)
        if (p) (void)hipFree(p);
    for (hipEvent_t e : L->ev)
        if (e) (void)hipEventDestroy(e);
    delete L;
}

template <typename T>
int dev_alloc(T** p, size_t bytes) {
    if (bytes == 0) bytes = 16;
    hipError_t e = hipMalloc((void**)p, bytes);
    if (e != hipSuccess) {
        *p = nullptr;
        (void)hipGetLastError();
        return fail(MOE_ENOMEM, "hipMalloc(%zu bytes) failed: %s", bytes, hipGetErrorString(e));
    }
    return MOE_OK;
}

int check_desc(const moe_desc* d, const moe_weights* w) {
    if (d->d_model <= 0 || d->n_experts <= 0 || d->d_ff <= 0 || d->top_k <= 0 || d->max_tokens <= 0)
        return fail(MOE_EINVAL, "sizes must be positive (d_model=%d n_experts=%d d_ff=%d top_k=%d max_tokens=%d)",
                    d->d_model, d->n_experts, d->d_ff, d->top_k, d->max_tokens);
    if (d->top_k > d->n_experts) return fail(MOE_EINVAL, "top_k=%d > n_experts=%d", d->top_k, d->n_experts);
    if (d->shared_d_ff < 0) return fail(MOE_EINVAL, "shared_d_ff < 0");
    if (d->profile != 0 && d->profile != 1) return fail(MOE_EINVAL, "profile must be 0 or 1");
    if (d->gate_clamp != 0 && d->gate_clamp != 1) return fail(MOE_EINVAL, "gate_clamp must be 0 or 1");
    if (d->gate_weighting != MOE_WEIGHT_SOFTMAX && d->gate_weighting != MOE_WEIGHT_RAW)
        return fail(MOE_EINVAL, "gate_weighting must be MOE_WEIGHT_SOFTMAX (0) or MOE_WEIGHT_RAW (1)");
    if (!w->w_router || !w->w_gate || !w->w_up || !w->w_down)
        return fail(MOE_EINVAL, "w_router, w_gate, w_up and w_down are required");
    const bool f32 = d->act_dtype == MOE_F32 && d->expert_dtype == MOE_F32;
    const bool bf = d->act_dtype == MOE_BF16 && d->expert_dtype == MOE_BF16;
    const bool i8 = d->act_dtype == MOE_BF16 && d->expert_dtype == MOE_I8;
    const bool i4 = d->act_dtype == MOE_BF16 && d->expert_dtype == MOE_I4;
    if (!(f32 || bf || i8 || i4))
        return fail(MOE_EUNSUPPORTED, "dtype pair (act=%d, expert=%d) not supported", d->act_dtype,
                    d->expert_dtype);
    if ((i8 || i4) && (!w->s_gate || !w->s_up || !w->s_down))
        return fail(MOE_EINVAL, "int8 and int4 experts need s_gate, s_up and s_down");
    if (d->shared_d_ff > 0 && (!w->w_shared_gate || !w->ws_gate || !w->ws_up || !w->ws_down))
        return fail(MOE_EINVAL, "shared expert needs w_shared_gate, ws_gate, ws_up and ws_down");
    if (d->n_experts > kMaxExperts) return fail(MOE_EUNSUPPORTED, "n_experts=%d > %d", d->n_experts, kMaxExperts);
    if (d->top_k > kMaxTopK) return fail(MOE_EUNSUPPORTED, "top_k=%d > %d", d->top_k, kMaxTopK);
    const int dm = f32 ? 64 : 128;
    if (d->d_model % dm || d->d_ff % 64)
        return fail(MOE_EUNSUPPORTED, "need d_model %% %d == 0 and d_ff %% 64 == 0 (d_model=%d d_ff=%d)", dm,
                    d->d_model, d->d_ff);
    if (i4 && d->d_ff % 128)
        return fail(MOE_EUNSUPPORTED, "int4 experts need d_ff %% 128 == 0 (d_ff=%d)", d->d_ff);
    if (d->shared_d_ff > 0) {
        if (!bf) return fail(MOE_EUNSUPPORTED, "a shared expert needs bf16 experts");
        if (d->shared_d_ff % d->d_ff)
            return fail(MOE_EUNSUPPORTED, "shared_d_ff=%d must be a multiple of d_ff=%d", d->shared_d_ff, d->d_ff);
        if (d->shared_d_ff / d->d_ff > kMaxVirtual)
            return fail(MOE_EUNSUPPORTED, "shared_d_ff / d_ff = %d > %d", d->shared_d_ff / d->d_ff, kMaxVirtual);
    }
    // all index arithmetic in the kernels is 32-bit on rows and slots
    const long long P = (long long)d->max_tokens * (d->top_k + (d->shared_d_ff / d->d_ff));
    if (P >= (1ll << 30)) return fail(MOE_EUNSUPPORTED, "max_tokens * slots too large (%lld)", P);
    return MOE_OK;
}

int scratch_on_device(int dev, char** out);

int create_impl(const moe_desc* desc, const moe_weights* w, moe_layer* L) {
    const moe_desc& d = *desc;
    L->desc = d;
    L->E = d.n_experts;
    L->V = d.shared_d_ff / d.d_ff;
    L->Et = L->E + L->V;
    L->kt = d.top_k + L->V;
    L->Ec = L->E + (d.shared_d_ff > 0 ? 1 : 0);
    L->has_bias = w->b_router != nullptr;
    HIP_TRY(hipGetDevice(&L->device));
    HIP_TRY(hipDeviceGetAttribute(&L->cus, hipDeviceAttributeMultiprocessorCount, L->device));
    {
        // the device address of the static scratch on this device, for moe_forward_noalloc
        char* sp;
        int rc0 = scratch_on_device(L->device, &sp);
        if (rc0) return rc0;
    }

    const size_t dm = d.d_model, F = d.d_ff, E = L->E, Et = L->Et;
    const bool f32 = d.expert_dtype == MOE_F32;
    const bool i8 = d.expert_dtype == MOE_I8;
    const bool i4 = d.expert_dtype == MOE_I4;
    // bytes per 2 weights (int4 packs two in a byte)
    const size_t esz2 = f32 ? 8 : (i8 ? 2 : (i4 ? 1 : 4));
    int rc;
    if ((rc = dev_alloc(&L->wr_t, (size_t)L->Ec * dm * 4))) return rc;
    if (!f32 && (rc = dev_alloc(&L->wr_planes, (size_t)3 * ((L->Ec + 15) / 16) * 16 * dm * 2))) return rc;
    if (L->has_bias && (rc = dev_alloc(&L->bias, E * 4))) return rc;
    if ((rc = dev_alloc(&L->wgu, Et * F * dm * esz2))) return rc;
    if ((rc = dev_alloc(&L->wdn, Et * F * dm * esz2 / 2))) return rc;
    if (i4) {
        // group scales: the up projection's in packed column order, the down projection's as given
        if ((rc = dev_alloc(&L->s_gate, E * (dm / 128) * 2 * F * 4))) return rc;
        if ((rc = dev_alloc(&L->s_down, E * (F / 128) * dm * 4))) return rc;
    }
    if (i8) {
        if ((rc = dev_alloc(&L->s_gate, E * F * 4))) return rc;
        if ((rc = dev_alloc(&L->s_up, E * F * 4))) return rc;
        if ((rc = dev_alloc(&L->s_down, E * dm * 4))) return rc;
    }
    const size_t T = d.max_tokens, P = T * L->kt;
    Work& ws = L->w;
    if ((rc = dev_alloc(&ws.counts, (Et + 1) * 4))) return rc;
    if ((rc = dev_alloc(&ws.offsets, (Et + 1) * 4))) return rc;
    if ((rc = dev_alloc(&ws.tile_start, (Et + 1) * 4))) return rc;
    if ((rc = dev_alloc(&ws.tile_start_h, (Et + 1) * 4))) return rc;
    if ((rc = dev_alloc(&ws.sorted_c, P * 4))) return rc;
    if ((rc = dev_alloc(&ws.gs, T * 4))) return rc;
    if ((rc = dev_alloc(&ws.ridx, T * d.top_k * 4))) return rc;
    if ((rc = dev_alloc(&ws.rw, T * d.top_k * 4))) return rc;
    {
        // the split decode gate's partial dots, or the MFMA gate's partial logits
        const size_t split = gate_split_workspace((int)std::min(T, (size_t)64), d.d_model, L->E, d.shared_d_ff > 0);
        const size_t mfma = f32 ? 0 : gate_mfma_workspace_max((int)T, L->E, d.shared_d_ff > 0);
        ws.gate_part_bytes = std::max(split, mfma);
        if ((rc = dev_alloc(&ws.gate_part, ws.gate_part_bytes))) return rc;
    }
    if ((rc = dev_alloc(&ws.scatter_work, scatter_wide_workspace((int)(T * d.top_k), L->E)))) return rc;
    // the tiled GEMMs work on padded rows: at most P + (bm - 1) + Et*bm of them for bm <= 256
    const size_t R = P + (size_t)256 * (Et + 1);
    if (!f32 && (rc = dev_alloc(&ws.xp, R * dm * 2))) return rc;
    if ((rc = dev_alloc(&ws.h, (f32 ? P : R) * F * (f32 ? 4 : 2)))) return rc;
    // combine buffer: one row per (token, slot, K split): 2 splits for large batches,
    // up to kStreamMaxSplit for batches the streaming kernels serve
    // (int8 and int4 layers: 4, so the tile-stream down projection can split K four ways at
    // ~64 rows per expert; 8-expert int8 layer T = 512: 0.96 -> 0.89 ms)
    L->ow_rows = std::max(P * (i8 || i4 ? 4 : 2), std::min(T, (size_t)kStreamMaxT) * L->kt * kStreamMaxSplit);
    if ((rc = dev_alloc(&ws.ow, L->ow_rows * dm * 4))) return rc;
    if (d.profile) {
        for (hipEvent_t& e : L->ev) HIP_TRY(hipEventCreate(&e));
        L->profiling = true;
    }

    hipStream_t s = nullptr;
    HIP_TRY(pack_router(w->w_router, d.shared_d_ff > 0 ? w->w_shared_gate : nullptr, d.d_model, L->E, L->wr_t, s));
    if (L->wr_planes)
        HIP_TRY(pack_router_planes(w->w_router, d.shared_d_ff > 0 ? w->w_shared_gate : nullptr, d.d_model, L->E,
                                   L->wr_planes, s));
    if (L->has_bias) HIP_TRY(hipMemcpyAsync(L->bias, w->b_router, E * 4, hipMemcpyDeviceToDevice, s));
    if (f32) {
        // fp32 experts keep the natural layout: [E][d][F] gate, [E][d][F] up, [E][F][d] down
        HIP_TRY(hipMemcpyAsync(L->wgu, w->w_gate, E * dm * F * 4, hipMemcpyDeviceToDevice, s));
        HIP_TRY(hipMemcpyAsync((char*)L->wgu + E * dm * F * 4, w->w_up, E * dm * F * 4, hipMemcpyDeviceToDevice, s));
        HIP_TRY(hipMemcpyAsync(L->wdn, w->w_down, E * F * dm * 4, hipMemcpyDeviceToDevice, s));
    } else if (i4) {
        HIP_TRY(pack_gu_i4((const uint8_t*)w->w_gate, (const uint8_t*)w->w_up, L->E, d.d_model, d.d_ff,
                           (uint8_t*)L->wgu, s));
        HIP_TRY(pack_dn_i4((const uint8_t*)w->w_down, L->E, d.d_ff, d.d_model, (uint8_t*)L->wdn, s));
        HIP_TRY(pack_scales_gu_i4(w->s_gate, w->s_up, L->E, d.d_model, d.d_ff, L->s_gate, s));
        HIP_TRY(hipMemcpyAsync(L->s_down, w->s_down, E * (F / 128) * dm * 4, hipMemcpyDeviceToDevice, s));
    } else if (i8) {
        HIP_TRY(pack_gu_i8((const int8_t*)w->w_gate, (const int8_t*)w->w_up, L->E, d.d_model, d.d_ff,
                           (int8_t*)L->wgu, s));
        HIP_TRY(pack_dn_i8((const int8_t*)w->w_down, L->E, d.d_ff, d.d_model, (int8_t*)L->wdn, s));
        HIP_TRY(hipMemcpyAsync(L->s_gate, w->s_gate, E * F * 4, hipMemcpyDeviceToDevice, s));
        HIP_TRY(hipMemcpyAsync(L->s_up, w->s_up, E * F * 4, hipMemcpyDeviceToDevice, s));
        HIP_TRY(hipMemcpyAsync(L->s_down, w->s_down, E * dm * 4, hipMemcpyDeviceToDevice, s));
    } else {
        HIP_TRY(pack_gu_bf16((const bf16_t*)w->w_gate, (const bf16_t*)w->w_up, L->E, d.d_model, d.d_ff,
                             (bf16_t*)L->wgu, d.d_ff, s));
        HIP_TRY(pack_dn_bf16((const bf16_t*)w->w_down, L->E, d.d_ff, d.d_model, (bf16_t*)L->wdn, s));
        // shared expert: slice v = columns [v*F, (v+1)*F) of ws_gate/ws_up and rows of ws_down
        for (int v = 0; v < L->V; ++v) {
            const size_t eo = (size_t)(L->E + v);
            HIP_TRY(pack_gu_bf16((const bf16_t*)w->ws_gate + (size_t)v * F, (const bf16_t*)w->ws_up + (size_t)v * F,
                                 1, d.d_model, d.d_ff, (bf16_t*)L->wgu + eo * 2 * F * dm, d.shared_d_ff, s));
            HIP_TRY(pack_dn_bf16((const bf16_t*)w->ws_down + (size_t)v * F * dm, 1, d.d_ff, d.d_model,
                                 (bf16_t*)L->wdn + eo * F * dm, s));
        }
    }
    HIP_TRY(hipStreamSynchronize(s));
    return MOE_OK;
}

// ---- the forward, shared by moe_forward and moe_forward_routed

// Checks common to both forward entry points (before any HIP call).
int check_call(const moe_layer* L, const void* x, int32_t T, void* y) {
    if (!L) return fail(MOE_EINVAL, "layer is NULL");
    if (T < 0 || T > L->desc.max_tokens) return fail(MOE_EINVAL, "T=%d outside [0, %d]", T, L->desc.max_tokens);
    if (T == 0) return MOE_OK;  // nothing to read or write; buffers may be empty
    if (!x || !y) return fail(MOE_EINVAL, "x and y are required");
    if (!aligned(x, 16) || !aligned(y, 16)) return fail(MOE_EINVAL, "x and y must be 16-byte aligned");
    return MOE_OK;
}

int check_device(const moe_layer* L) {
    int dev = -1;
    HIP_TRY(hipGetDevice(&dev));
    if (dev != L->device) return fail(MOE_EINVAL, "current device %d is not the layer's device %d", dev, L->device);
    return MOE_OK;
}

// Launch plan (host side, from T, k and the layer shape only):
//  - small batches (T <= 64; int8 and int4 weights: T <= 32) stream the weights: row tiles
//    of 16, 32 or 64 rows (int4: 16 or 32), sized so an active expert almost always fits one
//    tile, the down projection's K split so ~1024 workgroups run;
//  - larger batches of int8 and int4 weights (when both projections have whole 256-column
//    tiles) take the tile-stream GEMMs: row tiles in LDS, each wave streaming its weight
//    columns into registers (128-row tiles for int8, 64 when the experts average at most 32
//    rows; 64 for int4);
//  - other larger batches use the LDS-tiled MFMA GEMMs (256-row tiles for bf16 weights, 128
//    for int8, 64 for int4);
//  - in the last two the down projection's K is split when that fills the CUs better.
// Past this many routed assignments the scatter runs over many workgroups.
constexpr int kScatterWideMin = 4095;

struct Plan {
    bool streaming;
    int bm, ksplit, max_tiles;
    bool merge;         // tiled down projection of a multi-slice shared expert as one K loop
    bool weights_once;  // streaming: the busiest expert is expected to fit one row tile
    bool tstream;       // quantised weights past the streaming sizes: row tiles in LDS, weights
                        // streamed into registers (expert_tstream) instead of the LDS-tiled GEMMs
    int bm_h, max_tiles_h;  // the down projection's row tiling (H follows it); == bm, max_tiles
                            // but for the int4 tile-stream 80-row up tiles
};

Plan make_plan(const moe_layer* L, int T) {
    const moe_desc& d = L->desc;
    const bool f32 = d.expert_dtype == MOE_F32;
    const bool i8 = d.expert_dtype == MOE_I8;
    const bool i4 = d.expert_dtype == MOE_I4;
    const int k = d.top_k;
    // int8 and int4 weights at 33-64 tokens: the tile-stream kernels are faster (8-expert
    // 6144 x 16384 layer; int8 T = 64: 0.45 ms against 0.50 streaming, T = 24 and 32 stream
    // faster; int4 T = 48: 0.30 against 0.31 streaming); bf16 weights stream up to 64 (T = 64:
    // 0.50 against 0.58 ms tiled)
    const bool streaming = !f32 && T <= (i8 || i4 ? kStreamMaxT / 2 : kStreamMaxT);
    int bm, ksplit = 1, bm_h = 0;
    bool weights_once = true, tstream = false;
    if (f32) {
        bm = kBMf32;
    } else if (streaming) {
        // row tile: expected rows of the busiest expert (shared slices hold all T rows; routed
        // experts about twice their average), so an expert rarely needs a second tile
        const int need = L->V > 0 ? T : std::min(T, 2 * ((T * k + L->E - 1) / L->E));
        // int4 takes at most 32 rows a tile: its 64-row kernel holds too many registers
        // to hide memory latency, and re-streaming the (small) weights per tile costs less
        bm = need <= 16 ? 16 : (need <= 32 || i4 ? 32 : 64);
        weights_once = need <= bm;
        const int active = std::min(L->E, T * k) + L->V;
        const int groups = active * (d.d_model / 128);
        const int kstep = i4 ? 128 : 64;  // every split a whole number of weight steps
        while (ksplit < kStreamMaxSplit && groups * ksplit < 1024 && d.d_ff % (ksplit * 2 * kstep) == 0 &&
               (size_t)T * L->kt * ksplit * 2 <= L->ow_rows)
            ksplit *= 2;
    } else {
        // int8 and int4: the tile-stream kernels (8-expert 6144 x 16384 layer, against the
        // LDS-tiled ones: int8 T = 256 0.63 -> 0.57 ms, T = 1024 1.57 -> 1.40; int4 T = 256
        // 0.70 -> 0.61, T = 1024 1.89 -> 1.61) when both projections have whole 256-column
        // tiles
        // bf16 (no shared expert) while the experts average at most 128 rows: 128-row tiles up
        // to 96, 160-row ones past it (most experts then fit one tile, 160 being about three
        // standard deviations past 128 rows). 8-expert 4096 x 14336 layer against the
        // LDS-tiled 256-row tiles: T = 80-256 12-15% faster (T = 128 0.596 -> 0.512 ms), T =
        // 384 9%, 448 and 512 7-8% (160-row tiles; 128-row ones at 512: 0.69 -> 0.78 ms, most
        // experts spilling into a second tile that streams the weights again); T = 576 2%
        // slower. With uneven routing the average misleads (128-expert Zipf-biased layer: 5%
        // faster at T = 256, even at 1024, 5-9% slower at 2048-3072, where a few experts hold
        // most rows), so at most 4096 routed rows.
        const bool bf16_ts = !i8 && !i4 && L->V == 0 && (long long)T * k <= 128LL * L->E && (long long)T * k <= 4096;
        tstream = (i8 || i4 || bf16_ts) && (2 * d.d_ff) % 256 == 0 && d.d_model % 256 == 0;
        // bf16: 256-row tiles (the 256 x 256 workgroup tile reads the least LDS and L2 per MFMA
        // and outruns 128-row tiles even when most experts leave their last tile half empty);
        // int8: 128-row tiles, 64 when the experts average at most 24 rows (tile-stream: 32;
        // LDS-tiled T = 64 on the 8-expert layer: 0.48 against 0.51 ms; tile-stream T = 128
        // 0.48 against 0.49 ms, T = 256 0.66 against 0.57); int4: 64-row tiles (the
        // registers of a 128-row tile do not fit)
        bm = i4 ? 64 : (i8 ? ((long long)T * k <= (tstream ? 32LL : 24LL) * L->E ? 64 : 128)
                           : tstream ? ((long long)T * k <= 96LL * L->E ? 128 : 160) : 256);
        // int4 tile-stream with 41-72 rows per expert on average: 80-row up tiles, so nearly
        // every expert's weights stream once (not again for a ragged second tile of a few
        // rows), and 64-row down tiles (80-row down tiles measured within +-3% at T =
        // 176-288, and the smaller tiles give more workgroups): 8-expert 6144 x 16384 layer,
        // T = 256 0.608 -> 0.569 ms, T = 288 0.659 -> 0.623 ms
        if (tstream && i4 && (long long)T * k > 40LL * L->E && (long long)T * k <= 72LL * L->E) {
            bm = 80;
            bm_h = 64;
        }
        const int kq = i4 ? 128 : 64;  // every split a whole number of K steps
        // split the down projection's K (S = 2 or 4) when that fills the last round of
        // workgroups better: with W = tiles * column tiles * S workgroups and `slots` of them
        // at a time, the busy fraction is W / (rounds * slots); a split must gain 0.1 of it (the
        // partial rows cost combine traffic), keep K >= 2048 per split (4096 for a four-way
        // split: the 8-expert bf16 layer's 14336-wide down projection ran as fast split in two
        // as in four at T = 1024 and 2048, and the four-way split doubled the combine's
        // partial rows, T = 2048 1.559 -> 1.530 ms) and fit the combine buffer. The tile
        // count is its expectation under uniform routing: a routed expert
        // holds n ~ Binomial(T, k/E) rows (normal approximation) and needs
        // ceil(n / bm) = sum_j [n > j*bm] tiles; a shared slice holds all T rows.
        const double p_e = (double)k / L->E;
        const double mu = T * p_e, sd = std::sqrt(std::max(T * p_e * (1.0 - p_e), 1e-12));
        const int bmd = bm_h ? bm_h : bm;  // the down projection's tile height
        double tiles_e = 0.0;
        for (int j = 0; j * bmd < T; ++j) tiles_e += 0.5 * std::erfc((j * bmd + 0.5 - mu) / (sd * std::sqrt(2.0)));
        const double est_tiles = L->E * tiles_e + L->V * (double)((T + bmd - 1) / bmd);
        // down-projection column tiles and the workgroups one round runs: 256 columns, one per
        // CU (LDS-tiled) or two (tile-stream); the narrow int8 tile-stream down projection
        // takes 128 columns, four per CU with 64-row tiles and three with 128-row ones
        const bool narrow = tstream && i8 && tstream_narrow_down(T, k, L->E);
        const int nt_down = (d.d_model + (narrow ? 127 : 255)) / (narrow ? 128 : 256);
        const int slots = (narrow ? (bmd == 64 ? 4 : 3) : tstream ? 2 : 1) * L->cus;
        auto busy = [&](int S) {
            const double w = est_tiles * nt_down * S;
            return w / (std::ceil(w / slots) * slots);
        };
        double best = busy(1);
        for (int S = 2; S <= 4; S *= 2) {
            if (d.d_ff / S < (S > 2 ? 4096 : 2048) || d.d_ff % (S * kq) != 0 || (size_t)T * L->kt * S > L->ow_rows) break;
            if (busy(S) > best + 0.1) {
                best = busy(S);
                ksplit = S;
            }
        }
    }
    if ((size_t)T * L->kt * ksplit > L->ow_rows) ksplit = 1;  // never past the combine buffer
    // upper bound on sum_e ceil(n_e / bm) over experts with rows: one tile per active
    // expert, plus sum_e floor((n_e - 1) / bm) <= floor((P - 1) / bm) more for experts past
    // one tile (the streaming tile is sized to the expected busiest expert, not a bound)
    const int P = T * L->kt;
    const int max_tiles = std::min(L->Et, P) + (P - 1) / bm;
    if (!bm_h) bm_h = bm;
    const int max_tiles_h = std::min(L->Et, P) + (P - 1) / bm_h;
    // tiled down projection of a shared expert in several slices: the slices of a row tile
    // are summed in one K loop (one partial row per token instead of one per slice)
    const bool merge = !f32 && !streaming && !i8 && !i4 && L->V > 1 && ksplit == 1;
    return Plan{streaming, bm, ksplit, max_tiles, merge, weights_once, tstream, bm_h, max_tiles_h};
}

// Routers wider than 16 columns (experts + shared gate) at decode batch sizes: the split gate.
bool split_gate(const moe_layer* L, int T) {
    const bool wide_router = L->E + (L->V > 0 ? 1 : 0) > 16;
    const bool f32 = L->desc.expert_dtype == MOE_F32;
    return wide_router && gate_split_fits(T, L->desc.top_k) && (f32 || T <= kGateSplitMaxT);
}

// ---- the static scratch of the allocation-free forward (moe_forward_noalloc)
// One file-scope device array: every device the library runs on holds its own copy from
// the module's load until the process ends, shared by every layer and call on that device.
// In host code the name `scratch` is a host-side stand-in, not a device address: host code
// takes the array's device address once per device (hipGetSymbolAddress, at the first
// moe_layer_create on that device) and passes only that address to kernels.
constexpr size_t kScratchBytes = MOE_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's device address on `dev` (the current device), looked up on first use.
int scratch_on_device(int dev, char** out) {
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_EUNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        g_scratch_ptr[dev] = (char*)p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

// The workspace a forward of T tokens under plan pl reads and writes, laid out from `base`
// into *W (each piece on a 256-byte boundary); returns its size. base == nullptr: size only.
// Every byte a forward reads from it is written earlier in the same forward, so nothing
// needs clearing between calls.
size_t carve_work(const moe_layer* L, const Plan& pl, int T, char* base, Work* W) {
    const moe_desc& d = L->desc;
    const bool f32 = d.expert_dtype == MOE_F32;
    const size_t Et = L->Et, P = (size_t)T * L->kt, dm = d.d_model, F = d.d_ff;
    const size_t tiled_rows = (size_t)pl.max_tiles * pl.bm;  // padded rows of the tiled GEMM operands
    size_t off = 0;
    auto take = [&](size_t bytes) -> char* {
        char* p = base ? base + off : nullptr;
        off += (bytes + 255) / 256 * 256;
        return p;
    };
    Work w;
    w.counts = (int32_t*)take((Et + 1) * 4);
    w.offsets = (int32_t*)take((Et + 1) * 4);
    w.tile_start = (int32_t*)take((Et + 1) * 4);
    w.tile_start_h = (int32_t*)take((Et + 1) * 4);
    w.sorted_c = (int32_t*)take(P * 4);
    w.gs = (float*)take((size_t)T * 4);
    if (split_gate(L, T)) {
        w.gate_part_bytes = gate_split_workspace(T, d.d_model, L->E, L->V > 0);
        w.gate_part = (float*)take(w.gate_part_bytes);
    } else if (const size_t gm = gate_mfma_workspace(T, d.d_model, L->E, L->V > 0, !f32)) {
        w.gate_part_bytes = gm;
        w.gate_part = (float*)take(gm);
    }
    if (T * d.top_k > kScatterWideMin) w.scatter_work = (int32_t*)take(scatter_wide_workspace(T * d.top_k, L->E));
    if (!f32 && !pl.streaming) w.xp = (bf16_t*)take(tiled_rows * dm * 2);
    w.h = take((f32 || pl.streaming ? P : (size_t)pl.max_tiles_h * pl.bm_h) * F * (f32 ? 4 : 2));
    w.ow = (float*)take(P * pl.ksplit * dm * 4);
    if (W) *W = w;
    return off;
}

ScatterOut scatter_out(const Work& W, int32_t* counts, int32_t* offsets, int32_t* sorted) {
    return ScatterOut{W.counts, W.offsets, W.tile_start, W.sorted_c, counts, offsets, sorted};
}

// Scatter of a routing already in device memory (idx [T][k]).
int run_scatter(moe_layer* L, const Work& W, const int32_t* idx, int T, const Plan& pl, const ScatterOut& so,
                hipStream_t s) {
    const int k = L->desc.top_k;
    // many assignments: the scatter over many workgroups (three launches)
    if (T * k > kScatterWideMin)
        HIP_TRY(launch_scatter_wide(idx, T, L->E, k, L->V, pl.bm, so, W.scatter_work, s));
    else
        HIP_TRY(launch_scatter(idx, T, L->E, k, L->V, pl.bm, so, s));
    return MOE_OK;
}

// Expert compute and Gather once the scatter tables are on the device: the gathering
// of token rows for the tiled GEMMs, up, down, combine (with the per-stage events).
int run_experts(moe_layer* L, const Work& W, const void* x, int T, void* y, const float* topk_w, const float* gs,
                const Plan& pl, hipStream_t s) {
    const moe_desc& d = L->desc;
    const bool f32 = d.expert_dtype == MOE_F32;
    const bool i8 = d.expert_dtype == MOE_I8;
    const int wq = d.expert_dtype == MOE_I4 ? kWI4 : (i8 ? kWI8 : kWBf16);
    const int k = d.top_k;
    const bool prof = L->profiling;
    const GemmArgs a{W.tile_start, W.offsets, W.sorted_c, L->Et, L->kt, k, pl.max_tiles, pl.bm, pl.ksplit,
                     pl.merge ? 1 : 0, pl.weights_once ? 1 : 0, (const bf16_t*)x, W.xp, (bf16_t*)W.h, L->wgu, L->wdn,
                     L->s_gate, L->s_up, L->s_down, topk_w, gs, W.ow, d.d_model, d.d_ff, T,
                     pl.bm_h != pl.bm ? W.tile_start_h : W.tile_start, pl.bm_h};
    // the tiled GEMMs take the token rows already gathered into fragment order (and, with a
    // separate down tiling, launch_pack_a also fills its tile table)
    if (!f32 && !pl.streaming) HIP_TRY(launch_pack_a(a, s));
    if (prof) HIP_TRY(hipEventRecord(L->ev[2], s));
    if (f32) {
        GemmF32Args af{W.tile_start, W.offsets, W.sorted_c, L->Et, L->kt, k, pl.max_tiles,
                       (const float*)x, (float*)W.h, (const float*)L->wgu,
                       (const float*)L->wgu + (size_t)L->E * d.d_model * d.d_ff, (const float*)L->wdn,
                       topk_w, gs, W.ow, d.d_model, d.d_ff};
        HIP_TRY(launch_expert_up_f32(af, s));
        if (prof) HIP_TRY(hipEventRecord(L->ev[3], s));
        HIP_TRY(launch_expert_down_f32(af, s));
    } else if (pl.streaming) {
        HIP_TRY(launch_expert_up_stream(a, wq, s));
        if (prof) HIP_TRY(hipEventRecord(L->ev[3], s));
        HIP_TRY(launch_expert_down_stream(a, wq, s));
    } else if (pl.tstream) {
        HIP_TRY(launch_expert_up_tstream(a, wq, s));
        if (prof) HIP_TRY(hipEventRecord(L->ev[3], s));
        // the down projection on its own row tiling (the one H was written in)
        GemmArgs ad = a;
        ad.tile_start = a.tile_start_h;
        ad.bm = pl.bm_h;
        ad.max_tiles = pl.max_tiles_h;
        HIP_TRY(launch_expert_down_tstream(ad, wq, s));
    } else {
        HIP_TRY(launch_expert_up_tiled(a, wq, s));
        if (prof) HIP_TRY(hipEventRecord(L->ev[3], s));
        HIP_TRY(launch_expert_down_tiled(a, wq, s));
    }
    if (prof) HIP_TRY(hipEventRecord(L->ev[4], s));
    HIP_TRY(launch_combine(W.ow, T, (pl.merge ? k + 1 : L->kt) * pl.ksplit, L->kt * pl.ksplit, d.d_model, y, !f32,
                           s));
    if (prof) {
        HIP_TRY(hipEventRecord(L->ev[5], s));
        L->ran = true;
    }
    return MOE_OK;
}

// Checks of a forward's arguments (before any HIP call).
int check_forward(const moe_layer* L, const void* x, int32_t T, void* y, const moe_route_out* r) {
    int rc = check_call(L, x, T, y);
    if (rc || T == 0) return rc;
    if (!r || !r->topk_idx || !r->topk_w) return fail(MOE_EINVAL, "route, route->topk_idx and route->topk_w are required");
    const void* rp[] = {r->topk_idx, r->topk_w, r->expert_counts, r->expert_offsets, r->sorted_assign,
                        r->shared_gate};
    for (const void* q : rp)
        if (q && !aligned(q, 4)) return fail(MOE_EINVAL, "route outputs must be 4-byte aligned");
    return check_device(L);
}

// The forward on workspace W (the layer's own, or one carved out of the static scratch).
int run_forward(moe_layer* L, const Work& W, const void* x, int32_t T, void* y, const moe_route_out* r,
                const Plan& pl, hipStream_t s) {
    int rc;
    const moe_desc& d = L->desc;
    const bool f32 = d.expert_dtype == MOE_F32;
    const int k = d.top_k;
    float* gs = r->shared_gate ? r->shared_gate : W.gs;
    const bool prof = L->profiling;
    const ScatterOut so = scatter_out(W, r->expert_counts, r->expert_offsets, r->sorted_assign);
    if (prof) HIP_TRY(hipEventRecord(L->ev[0], s));

    // Routing for decode batches: up to 16 router columns, one workgroup reads the whole
    // router quickly enough (tiny batches fuse gate and scatter; larger ones run one gate
    // workgroup per token, then the scatter); more columns spread the router over many
    // workgroups (split gate, whose last launch also runs the scatter).
    const bool wide_router = L->E + (L->V > 0 ? 1 : 0) > 16;
    const int gflags = (L->V > 0 ? kGateShared : 0) | (d.gate_clamp ? kGateClamp : 0) |
                       (d.gate_weighting == MOE_WEIGHT_RAW ? kGateRaw : 0);
    if (!wide_router && gate_scatter_small_fits(T, d.d_model, L->E, L->V > 0, !f32)) {
        // tiny batch: both stages in one workgroup (the scatter stage then times as empty)
        HIP_TRY(launch_gate_scatter_small(x, !f32, L->wr_t, L->bias, T, d.d_model, L->E, gflags, k, r->topk_idx,
                                          r->topk_w, gs, L->V, pl.bm, so, s));
        if (prof) HIP_TRY(hipEventRecord(L->ev[1], s));
    } else if (split_gate(L, T)) {
        // decode batch: router dots on many workgroups, then top-k and scatter in one
        HIP_TRY(launch_gate_split(x, !f32, L->wr_t, L->bias, T, d.d_model, L->E, gflags, k, r->topk_idx,
                                  r->topk_w, gs, L->V, pl.bm, so, W.gate_part, s));
        if (prof) HIP_TRY(hipEventRecord(L->ev[1], s));
    } else {
        HIP_TRY(launch_gate(x, !f32, L->wr_t, L->wr_planes, L->bias, T, d.d_model, L->E, gflags, k, r->topk_idx,
                            r->topk_w, gs, W.gate_part, W.gate_part_bytes, s));
        if (prof) HIP_TRY(hipEventRecord(L->ev[1], s));
        if ((rc = run_scatter(L, W, r->topk_idx, T, pl, so, s))) return rc;
    }
    return run_experts(L, W, x, T, y, r->topk_w, gs, pl, s);
}

}  // namespace

extern "C" {

const char* moe_status_str(int status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
        case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: unsupported configuration";
        case MOE_ENOMEM: return "MOE_ENOMEM: device allocation failed";
        case MOE_EHIP: return "MOE_EHIP: HIP runtime error";
        default: return "unknown moe status";
    }
}

const char* moe_last_error(void) { return g_err; }

int moe_layer_create(const moe_desc* desc, const moe_weights* weights, moe_layer** out) {
    g_err[0] = 0;
    if (!out) return fail(MOE_EINVAL, "out is NULL");
    *out = nullptr;
    if (!desc || !weights) return fail(MOE_EINVAL, "desc and weights are required");
    int rc = check_desc(desc, weights);
    if (rc) return rc;
    moe_layer* L = new (std::nothrow) moe_layer();
    if (!L) return fail(MOE_ENOMEM, "host allocation failed");
    rc = create_impl(desc, weights, L);
    if (rc) {
        release(L);
        return rc;
    }
    *out = L;
    return MOE_OK;
}

int moe_forward(moe_layer* L, const void* x, int32_t T, void* y, const moe_route_out* r, void* stream) {
    g_err[0] = 0;
    int rc = check_forward(L, x, T, y, r);
    if (rc || T == 0) return rc;
    return run_forward(L, L->w, x, T, y, r, make_plan(L, T), (hipStream_t)stream);
}

int moe_forward_noalloc(moe_layer* L, const void* x, int32_t T, void* y, const moe_route_out* r, void* stream) {
    g_err[0] = 0;
    int rc = check_forward(L, x, T, y, r);
    if (rc || T == 0) return rc;
    // the same plan as moe_forward, so the two give the same results
    const Plan pl = make_plan(L, T);
    const size_t need = carve_work(L, pl, T, nullptr, nullptr);
    if (need > kScratchBytes)
        return fail(MOE_EINVAL,
                    "moe_forward_noalloc: T=%d on this layer needs %zu bytes of scratch; the static scratch "
                    "holds %zu (moe_forward takes any T up to max_tokens)", T, need, kScratchBytes);
    char* base = nullptr;
    if ((rc = scratch_on_device(L->device, &base))) return rc;
    Work W;
    carve_work(L, pl, T, base, &W);
    return run_forward(L, W, x, T, y, r, pl, (hipStream_t)stream);
}

int moe_forward_routed(moe_layer* L, const void* x, int32_t T, const int32_t* topk_idx, const float* topk_w,
                       const float* shared_gate, void* y, const moe_route_out* r, void* stream) {
    g_err[0] = 0;
    int rc = check_call(L, x, T, y);
    if (rc || T == 0) return rc;
    if (!topk_idx || !topk_w) return fail(MOE_EINVAL, "topk_idx and topk_w are required");
    if (L->V > 0 && !shared_gate) return fail(MOE_EINVAL, "a layer with a shared expert needs shared_gate");
    if (L->V == 0 && shared_gate) return fail(MOE_EINVAL, "shared_gate given but the layer has no shared expert");
    const void* ip[] = {topk_idx, topk_w, shared_gate, r ? r->expert_counts : nullptr,
                        r ? r->expert_offsets : nullptr, r ? r->sorted_assign : nullptr};
    for (const void* q : ip)
        if (q && !aligned(q, 4)) return fail(MOE_EINVAL, "routing inputs and outputs must be 4-byte aligned");
    if ((rc = check_device(L))) return rc;

    hipStream_t s = (hipStream_t)stream;
    const bool prof = L->profiling;
    const Plan pl = make_plan(L, T);
    const Work& W = L->w;
    const ScatterOut so = scatter_out(W, r ? r->expert_counts : nullptr, r ? r->expert_offsets : nullptr,
                                      r ? r->sorted_assign : nullptr);
    if (prof) HIP_TRY(hipEventRecord(L->ev[0], s));
    // the given routing, with ids outside [0, E) read as expert 0 at weight 0
    HIP_TRY(launch_route_in(topk_idx, topk_w, T * L->desc.top_k, L->E, W.ridx, W.rw, s));
    if (prof) HIP_TRY(hipEventRecord(L->ev[1], s));
    if ((rc = run_scatter(L, W, W.ridx, T, pl, so, s))) return rc;
    return run_experts(L, W, x, T, y, W.rw, shared_gate, pl, s);
}

int moe_set_profiling(moe_layer* L, int enable) {
    g_err[0] = 0;
    if (!L) return fail(MOE_EINVAL, "layer is NULL");
    if (enable != 0 && enable != 1) return fail(MOE_EINVAL, "enable must be 0 or 1");
    if (enable && !L->ev[0])
        for (hipEvent_t& e : L->ev) HIP_TRY(hipEventCreate(&e));
    L->profiling = enable != 0;
    return MOE_OK;
}

int moe_stage_times(moe_layer* L, float ms[5]) {
    g_err[0] = 0;
    if (!L || !ms) return fail(MOE_EINVAL, "layer and ms are required");
    if (!L->ran) return fail(MOE_EINVAL, "no forward has run with profiling on");
    HIP_TRY(hipEventSynchronize(L->ev[5]));
    for (int i = 0; i < 5; ++i) HIP_TRY(hipEventElapsedTime(&ms[i], L->ev[i], L->ev[i + 1]));
    return MOE_OK;
}

void moe_destroy(moe_layer* L) {
    if (!L) return;
    (void)hipDeviceSynchronize();
    release(L);
}

}  // extern "C"
