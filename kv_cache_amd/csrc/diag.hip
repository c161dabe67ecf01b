// Measurement helper, not a step of the method: reads the INT4 store of a
// hybrid cache with the decode kernel's access pattern (64-token tiles,
// 4 KiB of K codes, 1 KiB of K and of V scale/zero, 4 KiB of V codes, 128-bit
// buffer loads, two tiles in flight per wave, the same splits) and computes
// nothing but an XOR of what it read, so its time is the streaming-read time
// of those bytes on this GPU: the achievable rate the decode kernel is
// compared against. The XOR of all sink words is the XOR of every 32-bit
// word read (the n_q/64 leading tiles of each (b, g)), which a test checks.
#include "hq_internal.h"

namespace hq {
namespace {

constexpr int kDiagWaves = 4;

__global__ __launch_bounds__(256, 2) void k_diag_read_int4(const hq_cache c, uint32_t* sink, int nsq) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int bg = b * c.Hkv + g;
    const int n_q = c.counts[4 * bg + 1];
    const int nqt = (n_q + kTile - 1) / kTile;
    const int v0 = s * nqt / nsq, v1 = (s + 1) * nqt / nsq;
    const QSpan qs = q_span(c, bg);
    const int wq = qs.tiles * kTileBytesQ;
    const __amdgpu_buffer_rsrc_t rkc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const uint8_t*>(c.k_codes) + (size_t)qs.tile0 * kTileBytesQ), (short)0, wq, 0x00020000);
    const __amdgpu_buffer_rsrc_t rvc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const uint8_t*>(c.v_codes) + (size_t)qs.tile0 * kTileBytesQ), (short)0, wq, 0x00020000);
    const __amdgpu_buffer_rsrc_t rkm = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const uint8_t*>(c.k_meta) + (size_t)qs.tile0 * 1024), (short)0, qs.tiles * 1024,
        0x00020000);
    const __amdgpu_buffer_rsrc_t rvm = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const uint8_t*>(c.v_meta) + (size_t)qs.tile0 * 1024), (short)0, qs.tiles * 1024,
        0x00020000);
    const int voff = lane * 16;
    auto ld = [&](const __amdgpu_buffer_rsrc_t& r, int soff) {
        return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kLoadNT));
    };
    uint4 acc = make_uint4(0, 0, 0, 0);
    auto fold = [&](const uint4& x) {
        acc.x ^= x.x;
        acc.y ^= x.y;
        acc.z ^= x.z;
        acc.w ^= x.w;
    };
    for (int v = v0 + wave; v < v1; v += 2 * kDiagWaves) {
        const int v2 = v + kDiagWaves < v1 ? v + kDiagWaves : v;
        uint4 t[2][10];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int tv = k ? v2 : v;
#pragma unroll
            for (int i = 0; i < 4; ++i) t[k][i] = ld(rkc, tv * kTileBytesQ + i * 1024);
            t[k][4] = ld(rkm, tv * 1024);
            t[k][5] = ld(rvm, tv * 1024);
#pragma unroll
            for (int i = 0; i < 4; ++i) t[k][6 + i] = ld(rvc, tv * kTileBytesQ + i * 1024);
        }
#pragma unroll
        for (int i = 0; i < 10; ++i) fold(t[0][i]);
        if (v2 != v) {  // a lone last tile is loaded twice but counted once
#pragma unroll
            for (int i = 0; i < 10; ++i) fold(t[1][i]);
        }
    }
    const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    sink[(((size_t)bg * nsq + s) * 4 + wave) * 64 + lane] = x;
}

// Largest relative error of the hardware base-2 exponential (v_exp_f32, the
// instruction the probe's pass 1 takes 2^f with) against the fp64 exponential
// over the fp32 inputs with order keys k0 .. k0 + n - 1 (the key of x is its
// bit pattern for x >= 0, minus the pattern of |x| for x < 0, so consecutive
// keys are consecutive fp32 values). One result per workgroup.
__global__ __launch_bounds__(256) void k_diag_exp2_error(int32_t k0, int64_t n, double* out) {
    __shared__ double red[4];
    double mx = 0.0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int32_t key = k0 + (int32_t)i;
        const uint32_t bits = key >= 0 ? (uint32_t)key : ((uint32_t)(-(int64_t)key) | 0x80000000u);
        const float x = __uint_as_float(bits);
        const double ref = exp2((double)x);
        const double e = (double)__builtin_amdgcn_exp2f(x);
        mx = fmax(mx, fabs(e - ref) / ref);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
}

}  // namespace

hipError_t launch_diag_exp2_error(int32_t k0, int64_t n, double* out, int nblocks, hipStream_t s) {
    k_diag_exp2_error<<<nblocks, 256, 0, s>>>(k0, n, out);
    return hipGetLastError();
}

size_t diag_sink_bytes(const hq_cache& c, int32_t tps) {
    return (size_t)c.B * c.Hkv * decode_nsq(c, tps) * 4 * 64 * sizeof(uint32_t);
}

hipError_t launch_diag_read_int4(const hq_cache& c, void* sink, int32_t tps, hipStream_t s) {
    const int nsq = decode_nsq(c, tps);
    k_diag_read_int4<<<dim3(nsq, c.Hkv, c.B), 256, 0, s>>>(c, static_cast<uint32_t*>(sink), nsq);
    return hipGetLastError();
}

}  // namespace hq
