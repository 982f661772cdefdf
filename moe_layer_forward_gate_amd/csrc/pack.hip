// Create-time repacking of the caller's weights into the kernels' layouts.
//
// [0539edu §3.1] weights are reorganised once, expert by expert, into one
// contiguous block per expert, and [hotelren §3.1] transposed to output-major
// ([out][in]) so a GEMM reads each output column's inputs contiguously. Here the
// target is the MFMA fragment order read by the expert GEMMs:
//   bf16 gate/up: [Et][2F/16][d/32][64 lanes][8]; packed 16-column block nb is
//                 gate columns 16*(nb/2).. when nb is even, up columns when odd;
//                 lane l, element v = column 16*(nb/2) + l%16, K row 32*ks + 8*(l/16) + v
//   bf16 down:    [Et][d/16][F/32][64][8], column nb*16 + l%16 of W_down
//   int8:         the same with 64 K rows per block and 16 bytes per lane,
//                 bytes 0-7 from the block's first 32 rows, bytes 8-15 the next 32
//   int4:         the same with 128 K rows (one scale group) per block, four
//                 words per lane, one per 32 rows (see pack_i4_kernel)
// and the router weight transposed to [Ec][d] (row E = the shared-expert gate).
// One thread writes one 16-byte lane chunk; runs once per layer.
#include "common.h"

namespace moe {
namespace {

__global__ void pack_router_kernel(const float* wr, const float* wsg, int d, int E, int Ec, float* out) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)Ec * d) return;
    const int e = (int)(i / d), k = (int)(i - (size_t)e * d);
    out[i] = e < E ? wr[(size_t)k * E + e] : wsg[k];
}

// Exact three-way split of an fp32 value into bf16 planes (round to nearest at each
// step; the remainders are exact in fp32 and the last one fits 8 bits).
__device__ __forceinline__ void split3(float v, bf16_t& hi, bf16_t& mid, bf16_t& lo) {
    hi = f32_to_bf16(v);
    const float r1 = v - bf16_to_f32(hi);
    mid = f32_to_bf16(r1);
    const float r2 = r1 - bf16_to_f32(mid);
    lo = f32_to_bf16(r2);
}

__global__ void pack_router_planes_kernel(const float* wr, const float* wsg, int d, int E, int Ec, int NB,
                                          bf16_t* out) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;  // one per (column, k)
    if (i >= (size_t)NB * 16 * d) return;
    const int col = (int)(i / d), k = (int)(i - (size_t)col * d);
    const float v = col < E ? wr[(size_t)k * E + col] : (col < Ec ? wsg[k] : 0.0f);
    bf16_t p[3];
    split3(v, p[0], p[1], p[2]);
    const int nb = col / 16, ks = k / 32, kin = k % 32;
    const int lane = col % 16 + 16 * (kin / 8);
    const size_t plane = (size_t)NB * (d / 32) * 64 * 8;
    const size_t off = (((size_t)nb * (d / 32) + ks) * 64 + lane) * 8 + kin % 8;
    out[off] = p[0];
    out[plane + off] = p[1];
    out[2 * plane + off] = p[2];
}

// src element (e, k, n) at src + e*K*ld + k*ld + n; for gate/up the packed column
// block nb reads src0 (gate) or src1 (up) at column 16*(nb/2).
template <typename T, int KPB>  // KPB: K rows per packed block (32 bf16, 64 int8)
__global__ void pack_kernel(const T* src0, const T* src1, int E, int K, int N, int64_t ld, bool gu, T* dst) {
    constexpr int PER = 16 / sizeof(T);  // elements per lane chunk
    const int NB = gu ? 2 * N / 16 : N / 16;
    const int KB = K / KPB;
    const size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t total = (size_t)E * NB * KB * 64;
    if (q >= total) return;
    const int ln = (int)(q % 64);
    size_t rest = q / 64;
    const int kb = (int)(rest % KB);
    rest /= KB;
    const int nb = (int)(rest % NB);
    const int e = (int)(rest / NB);
    const T* src = (gu && (nb & 1)) ? src1 : src0;
    const int n = (gu ? (nb / 2) : nb) * 16 + ln % 16;
    T v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int k = kb * KPB + (j / 8) * 32 + 8 * (ln / 16) + (j % 8);
        v[j] = src[(size_t)e * K * ld + (size_t)k * ld + n];
    }
    uint4 out;
    __builtin_memcpy(&out, v, 16);
    reinterpret_cast<uint4*>(dst)[q] = out;
}

template <typename T, int KPB>
hipError_t launch_pack(const T* s0, const T* s1, int E, int K, int N, int64_t ld, bool gu, T* dst, hipStream_t s) {
    const int NB = gu ? 2 * N / 16 : N / 16;
    const size_t total = (size_t)E * NB * (K / KPB) * 64;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL((pack_kernel<T, KPB>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, s0, s1, E, K,
                       N, ld, gu, dst);
    return hipGetLastError();
}

// int4: one thread per 16-byte lane chunk of a 1 KB block (16 columns x 128 K rows,
// one scale group). Source: two values per byte along K, low nibble = even row, 4-bit
// two's complement; packed: word s of lane l holds column l%16, K rows
// 128*kb + 32*s + 8*(l/16) + r for r = 0, 2, 4, 6 in nibbles 0-3 and r = 1, 3, 5, 7 in
// nibbles 4-7, as codes q + 8.
__global__ void pack_i4_kernel(const uint8_t* src0, const uint8_t* src1, int E, int K, int N, bool gu, uint32_t* dst) {
    const int NB = gu ? 2 * N / 16 : N / 16;
    const int KB = K / 128;
    const size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t total = (size_t)E * NB * KB * 64;
    if (q >= total) return;
    const int ln = (int)(q % 64);
    size_t rest = q / 64;
    const int kb = (int)(rest % KB);
    rest /= KB;
    const int nb = (int)(rest % NB);
    const int e = (int)(rest / NB);
    const uint8_t* src = ((gu && (nb & 1)) ? src1 : src0) + (size_t)e * (K / 2) * N;
    const int n = (gu ? (nb / 2) : nb) * 16 + ln % 16;
    uint32_t out[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int k0 = kb * 128 + 32 * w + 8 * (ln / 16);
        uint32_t word = 0;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int k = k0 + r;
            const uint32_t code = ((src[(size_t)(k / 2) * N + n] >> (4 * (k & 1))) + 8u) & 15u;  // (q + 8) mod 16
            const int nib = (r & 1) ? 4 + r / 2 : r / 2;
            word |= code << (4 * nib);
        }
        out[w] = word;
    }
    reinterpret_cast<uint4*>(dst)[q] = uint4{out[0], out[1], out[2], out[3]};
}

// Up-projection group scales [E][d/128][F] (gate, up) into [E][d/128][2F] in packed
// column order (block nb: gate columns 16*(nb/2).. when even, up when odd).
__global__ void pack_scales_gu_kernel(const float* sg, const float* su, int E, int G, int F, float* dst) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)E * G * 2 * F) return;
    const int p = (int)(i % (2 * F));
    const size_t eg = i / (2 * F);
    const int nb = p / 16;
    const int n = (nb / 2) * 16 + p % 16;
    dst[i] = ((nb & 1) ? su : sg)[eg * F + n];
}

hipError_t launch_pack_i4(const uint8_t* s0, const uint8_t* s1, int E, int K, int N, bool gu, uint8_t* dst,
                          hipStream_t s) {
    if (K % 128) return hipErrorInvalidValue;
    const int NB = gu ? 2 * N / 16 : N / 16;
    const size_t total = (size_t)E * NB * (K / 128) * 64;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_i4_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, s0, s1, E, K, N, gu,
                       reinterpret_cast<uint32_t*>(dst));
    return hipGetLastError();
}

}  // namespace

hipError_t pack_gu_i4(const uint8_t* wg, const uint8_t* wu, int E, int d, int F, uint8_t* dst, hipStream_t s) {
    return launch_pack_i4(wg, wu, E, d, F, true, dst, s);
}
hipError_t pack_dn_i4(const uint8_t* wd, int E, int F, int d, uint8_t* dst, hipStream_t s) {
    return launch_pack_i4(wd, wd, E, F, d, false, dst, s);
}
hipError_t pack_scales_gu_i4(const float* sg, const float* su, int E, int d, int F, float* dst, hipStream_t s) {
    const size_t n = (size_t)E * (d / 128) * 2 * F;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_scales_gu_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, sg, su, E, d / 128,
                       F, dst);
    return hipGetLastError();
}

hipError_t pack_router(const float* wr, const float* wsg, int d, int E, float* wr_t, hipStream_t s) {
    const int Ec = E + (wsg ? 1 : 0);
    const size_t n = (size_t)Ec * d;
    hipLaunchKernelGGL(pack_router_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, wr, wsg, d, E, Ec,
                       wr_t);
    return hipGetLastError();
}

hipError_t pack_router_planes(const float* wr, const float* wsg, int d, int E, bf16_t* planes, hipStream_t s) {
    const int Ec = E + (wsg ? 1 : 0);
    const int NB = (Ec + 15) / 16;
    const size_t n = (size_t)NB * 16 * d;
    hipLaunchKernelGGL(pack_router_planes_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, wr, wsg, d, E,
                       Ec, NB, planes);
    return hipGetLastError();
}

hipError_t pack_gu_bf16(const bf16_t* wg, const bf16_t* wu, int E, int d, int F, bf16_t* dst, int64_t src_ld,
                        hipStream_t s) {
    return launch_pack<bf16_t, 32>(wg, wu, E, d, F, src_ld, true, dst, s);
}
hipError_t pack_dn_bf16(const bf16_t* wd, int E, int F, int d, bf16_t* dst, hipStream_t s) {
    return launch_pack<bf16_t, 32>(wd, wd, E, F, d, d, false, dst, s);
}
hipError_t pack_gu_i8(const int8_t* wg, const int8_t* wu, int E, int d, int F, int8_t* dst, hipStream_t s) {
    return launch_pack<int8_t, 64>(wg, wu, E, d, F, F, true, dst, s);
}
hipError_t pack_dn_i8(const int8_t* wd, int E, int F, int d, int8_t* dst, hipStream_t s) {
    return launch_pack<int8_t, 64>(wd, wd, E, F, d, d, false, dst, s);
}

}  // namespace moe
