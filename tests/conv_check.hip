// Test-only device code: the gfx950 hardware conversions the kernels use,
// run side by side with the software definitions the kernels carry
// (epx_device.h), over every input.  Built into tests/libconvcheck.so by
// conv_check.py; loaded by tests/test_gpu_conversions.py.
//
// Each check counts, per input class, the inputs seen and those on which the
// two sides differ (bit for bit), and keeps the first differing inputs.
#include "epx_device.h"

using namespace epx;

namespace {

constexpr int kKeep = 8;  // differing inputs kept per class

struct Tally {
    unsigned long long* counts;  // [classes][2]: inputs, mismatches
    uint32_t* first;             // [classes][kKeep] differing inputs (unordered)
    uint32_t* nfirst;            // [classes] how many slots of `first` are taken
};

// Per-thread tallies: inputs seen and differing per class, and the thread's
// first differing input per class (reported once, at the end).
struct Local {
    unsigned long long seen[4] = {0, 0, 0, 0}, bad[4] = {0, 0, 0, 0};
    uint32_t first[4] = {0, 0, 0, 0};
};

__device__ __forceinline__ void note(Local& l, int cls, bool differ, uint32_t input) {
    l.seen[cls] += 1;
    if (differ) {
        if (l.bad[cls] == 0) l.first[cls] = input;
        l.bad[cls] += 1;
    }
}

__device__ void flush(const Tally& t, int classes, const Local& l) {
    for (int c = 0; c < classes; ++c) {
        if (l.seen[c]) atomicAdd(&t.counts[2 * c], l.seen[c]);
        if (l.bad[c]) {
            atomicAdd(&t.counts[2 * c + 1], l.bad[c]);
            const uint32_t slot = atomicAdd(&t.nfirst[c], 1u);
            if (slot < (uint32_t)kKeep) t.first[c * kKeep + slot] = l.first[c];
        }
    }
}

// E2M1 encode (v_cvt_scalef32_pk_fp4_f32, scale 1, low nibble) against
// e2m1_encode.  Classes: 0 finite, 1 infinite, 2 NaN.
__global__ void k_e2m1_encode(Tally t, uint64_t begin, uint64_t n) {
    Local l;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const uint32_t u = (uint32_t)(begin + i);
        const float f = __uint_as_float(u);
        const uint32_t hw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, f, 0.0f, 1.0f, 0) & 0xFu;
        const uint32_t sw = e2m1_encode(f);
        const uint32_t a = u & 0x7FFFFFFFu;
        const int cls = a < 0x7F800000u ? 0 : (a == 0x7F800000u ? 1 : 2);
        note(l, cls, hw != sw, u);
    }
    flush(t, 3, l);
}

// E4M3 encode (v_cvt_pk_fp8_f32, low byte) against e4m3_signed.  Classes:
// 0 finite with |v| <= 464, 1 finite with |v| > 464, 2 infinite, 3 NaN.
__global__ void k_e4m3_encode(Tally t, uint64_t begin, uint64_t n) {
    Local l;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const uint32_t u = (uint32_t)(begin + i);
        const float f = __uint_as_float(u);
        const uint32_t hw = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f, 0.0f, 0, false) & 0xFFu;
        const uint32_t a = u & 0x7FFFFFFFu;
        const int cls = a >= 0x7F800000u ? (a == 0x7F800000u ? 2 : 3) : (__uint_as_float(a) <= 464.0f ? 0 : 1);
        const uint32_t sw = cls <= 1 ? e4m3_signed(f) : 0xFFFFu;  // no software code outside the finite range
        note(l, cls, hw != sw, u);
    }
    flush(t, 4, l);
}

// bf16 rounding (v_cvt_pk_bf16_f32, low half) against bf16_rne_bits.
// Classes: 0 finite, 1 infinite, 2 NaN.
__global__ void k_bf16(Tally t, uint64_t begin, uint64_t n) {
    Local l;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const uint32_t u = (uint32_t)(begin + i);
        const float f = __uint_as_float(u);
        const uint32_t hw = pack_bf16x2(f, 0.0f) & 0xFFFFu;
        const uint32_t sw = bf16_rne_bits(f);
        const uint32_t a = u & 0x7FFFFFFFu;
        const int cls = a < 0x7F800000u ? 0 : (a == 0x7F800000u ? 1 : 2);
        note(l, cls, hw != sw, u);
    }
    flush(t, 3, l);
}

// E2M1 decode (v_cvt_scalef32_pk_f32_fp4, scale 1) of every byte in every
// byte position: out[(byte * 4 + sel) * 2 + {0, 1}] = float bits of the low-
// and high-nibble values; ref the same from e2m1_decode.
template <int SEL>
__device__ void decode_sel(uint32_t byte, uint32_t* out, uint32_t* ref) {
    const f32x2_t v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(byte << (8 * SEL), 1.0f, SEL);
    out[(byte * 4 + SEL) * 2] = __float_as_uint(v.x);
    out[(byte * 4 + SEL) * 2 + 1] = __float_as_uint(v.y);
    ref[(byte * 4 + SEL) * 2] = __float_as_uint(e2m1_decode(byte & 0xFu));
    ref[(byte * 4 + SEL) * 2 + 1] = __float_as_uint(e2m1_decode(byte >> 4));
}

__global__ void k_e2m1_decode(uint32_t* out, uint32_t* ref) {
    const uint32_t byte = threadIdx.x;  // 256 threads
    decode_sel<0>(byte, out, ref);
    decode_sel<1>(byte, out, ref);
    decode_sel<2>(byte, out, ref);
    decode_sel<3>(byte, out, ref);
}

// E4M3 decode (v_cvt_f32_fp8, byte 0) of every byte: out[c] = float bits of
// the hardware value, ref[c] = e4m3_decode_signed(c).
__global__ void k_e4m3_decode(uint32_t* out, uint32_t* ref) {
    const uint32_t c = threadIdx.x;  // 256 threads
    out[c] = __float_as_uint(__builtin_amdgcn_cvt_f32_fp8((int)c, 0));
    ref[c] = __float_as_uint(e4m3_decode_signed(c));
}

// The same conversion with the scale operand set to a block scale
// bs = e4m3(sc) * float(rowscale), against e2m1_decode(code) * bs, for
// every code, every finite E4M3 scale byte and every finite bf16 rowscale.
// Input id = code << 24 | sc << 16 | rowscale bits.  Classes: 0 bs and the
// product normal or zero, 1 product subnormal, 2 bs subnormal.
__global__ void k_e2m1_decode_scaled(Tally t) {
    Local l;
    const uint32_t code = blockIdx.y, sc = blockIdx.z;
    if ((sc & 0x7Fu) == 0x7Fu) return;  // the E4M3 NaN codes
    for (uint32_t rs = blockIdx.x * blockDim.x + threadIdx.x; rs < 65536u; rs += gridDim.x * blockDim.x) {
        if (((rs >> 7) & 0xFFu) == 0xFFu) continue;  // bf16 infinities and NaNs
        const float bs = e4m3_decode_signed(sc) * bf16_lo(rs);
        const f32x2_t pair = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code | (code << 4), bs, 0);
        const float hw = pair.x;
        const float sw = e2m1_decode(code) * bs;
        const uint32_t pb = __float_as_uint(sw) & 0x7FFFFFFFu, bb = __float_as_uint(bs) & 0x7FFFFFFFu;
        const int cls = (bb != 0u && bb < 0x00800000u) ? 2 : ((pb != 0u && pb < 0x00800000u) ? 1 : 0);
        note(l, cls, __float_as_uint(hw) != __float_as_uint(sw), (code << 24) | (sc << 16) | rs);
    }
    flush(t, 3, l);
}

// The software routines on a list of inputs (for comparison with the CPU
// oracle at every rounding boundary): E2M1 code, signed E4M3 code, bf16 bits.
__global__ void k_eval_sw(const float* in, int n, uint8_t* e2m1, uint8_t* e4m3, uint16_t* bf16) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const float f = in[i];
    e2m1[i] = (uint8_t)e2m1_encode(f);
    e4m3[i] = (uint8_t)e4m3_signed(f);
    bf16[i] = (uint16_t)bf16_rne_bits(f);
}

Tally tally(void* counts, void* first, void* nfirst) {
    return Tally{static_cast<unsigned long long*>(counts), static_cast<uint32_t*>(first),
                 static_cast<uint32_t*>(nfirst)};
}

}  // namespace

extern "C" {

// kind 0: E2M1 encode, 1: E4M3 encode, 2: bf16 rounding; float patterns
// [begin, begin + n).  counts: u64 [4][2], first: u32 [4][8], nfirst: u32 [4],
// all device memory, accumulated across calls.
int conv_check_encode(int kind, uint64_t begin, uint64_t n, void* counts, void* first, void* nfirst, void* stream) {
    const Tally t = tally(counts, first, nfirst);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid(4096), block(256);
    if (kind == 0) hipLaunchKernelGGL(k_e2m1_encode, grid, block, 0, st, t, begin, n);
    else if (kind == 1) hipLaunchKernelGGL(k_e4m3_encode, grid, block, 0, st, t, begin, n);
    else if (kind == 2) hipLaunchKernelGGL(k_bf16, grid, block, 0, st, t, begin, n);
    else return -1;
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

// out, ref: u32 [256 * 4 * 2] device memory.
int conv_check_e2m1_decode(void* out, void* ref, void* stream) {
    hipLaunchKernelGGL(k_e2m1_decode, dim3(1), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint32_t*>(out), static_cast<uint32_t*>(ref));
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

// out, ref: u32 [256] device memory.
int conv_check_e4m3_decode(void* out, void* ref, void* stream) {
    hipLaunchKernelGGL(k_e4m3_decode, dim3(1), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint32_t*>(out), static_cast<uint32_t*>(ref));
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

int conv_check_e2m1_decode_scaled(void* counts, void* first, void* nfirst, void* stream) {
    hipLaunchKernelGGL(k_e2m1_decode_scaled, dim3(64, 16, 256), dim3(256), 0, static_cast<hipStream_t>(stream),
                       tally(counts, first, nfirst));
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

int conv_eval_sw(const void* in, int n, void* e2m1, void* e4m3, void* bf16, void* stream) {
    if (n <= 0) return 0;
    hipLaunchKernelGGL(k_eval_sw, dim3((n + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const float*>(in), n, static_cast<uint8_t*>(e2m1), static_cast<uint8_t*>(e4m3),
                       static_cast<uint16_t*>(bf16));
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
