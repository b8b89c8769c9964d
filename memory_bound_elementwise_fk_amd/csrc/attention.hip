// attention.hip -- launcher of the FlashAttention forward kernel
// (attention_kernels.hpp).
#include <cmath>

#include "attention_kernels.hpp"
#include "launch.hpp"

namespace fk {

int64_t attention_head_dim() { return kAttnD; }

// workgroups of the 4-wave shape (the most the kernel is launched with)
int64_t attention_workgroups(int64_t B, int64_t H, int64_t T) {
    return (T + kAttnBQMin - 1) / kAttnBQMin * B * H;
}

template <int NW>
static const void* attention_kernel(Dtype dt, bool wide) {
    return dt == kF16
               ? (wide ? reinterpret_cast<const void*>(&attention_fwd_kernel<MmaF16, true, NW>)
                       : reinterpret_cast<const void*>(&attention_fwd_kernel<MmaF16, false, NW>))
               : (wide ? reinterpret_cast<const void*>(&attention_fwd_kernel<MmaBF16, true, NW>)
                       : reinterpret_cast<const void*>(&attention_fwd_kernel<MmaBF16, false, NW>));
}

// heads per group of the kernel's workgroup order: 1 for full attention, up
// to 4 for causal, a divisor of B H / 8; 0 when B H is not a multiple of 8
static int64_t attention_head_group(int64_t BH, int causal) {
    if (BH % 8 != 0) return 0;
    int64_t g = causal ? 4 : 1;
    while ((BH / 8) % g != 0) --g;
    return g;
}

hipError_t launch_attention_fwd(const void* q, const void* k, const void* v, void* o, int64_t B,
                                int64_t H, int64_t T, const int64_t* strides, int causal,
                                Dtype dt, hipStream_t s) {
    AttnArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.o = static_cast<uint16_t*>(o);
    a.B = B;
    a.H = H;
    a.T = T;
    a.qb = strides[0]; a.qh = strides[1]; a.qt = strides[2];
    a.kb = strides[3]; a.kh = strides[4]; a.kt = strides[5];
    a.vb = strides[6]; a.vh = strides[7]; a.vt = strides[8];
    a.ob = strides[9]; a.oh = strides[10]; a.ot = strides[11];
    a.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(double(kAttnD)));
    a.causal = causal;
    a.hgroup = attention_head_group(B * H, causal);
    // 8 waves per workgroup (one per CU) when that still gives every CU at
    // least four workgroups, else 4 (two per CU). Measured on B4 H32 (8 / 4
    // waves): full T1024 0.086 / 0.084 ms, T2048 0.269 / 0.281 ms, T4096
    // 1.027 / 1.075 ms; causal T1024 0.065 / 0.059 ms, T2048 0.163 / 0.168
    // ms, T4096 0.575 / 0.595 ms. With fewer rounds the 256-query
    // workgroups (causal: of different lengths) balance worse across the
    // CUs than 128-query ones.
    const int cus = device_cus();
    const int64_t nwg8 = (T + kAttnBQ<8> - 1) / kAttnBQ<8> * B * H;
    const bool w8 = cus > 0 && nwg8 >= 4 * int64_t(cus);
    // <= 2^23, checked by the caller
    const int64_t nwg = w8 ? nwg8 : attention_workgroups(B, H, T);
    void* args[] = {&a};
    // a lane's source offsets within a 64-key block fit 32 bits unless the
    // key strides are enormous (then the 64-bit variant)
    const int64_t lim = (int64_t(1) << 31) - kAttnD;
    const bool wide = a.kt > lim / kAttnBC || a.vt > lim / kAttnBC;
    const void* fn = w8 ? attention_kernel<8>(dt, wide) : attention_kernel<4>(dt, wide);
    return hipLaunchKernel(fn, dim3(static_cast<unsigned>(nwg)), dim3((w8 ? 8 : 4) * kWave), args,
                           0, s);
}

}  // namespace fk
