// gfx950 kernels for ragged recurrent-state checkpoints ("dasc: Decay-Aware
// State Compression for Hybrid Linear-Attention Serving", §4.1-§4.2 and
// App. B): pack the retained units of active slots into a flat checkpoint
// buffer, and restore a checkpoint into private slots with the omitted units
// zero-filled.  Both are pure byte movement, so they are written as 16-byte
// vector streams: grid.y = (src, dst) pair, grid.x = 4 KiB-per-wave chunks of
// that pair's bytes, four 16-byte vectors in flight per lane, nontemporal
// loads and stores (each byte is touched once).  The ragged index arithmetic
// (vector -> unit, unit -> layer) uses precomputed magic-number division and
// a binary search over the L+1 layer offsets held in LDS.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "hla.h"
#include "hla_device.h"
#include "hla_internal.h"

namespace hla {

constexpr int kCopyThreads = 256;
constexpr int kCopyVecs = 4;  // 16-byte vectors per lane per block
constexpr int kMaxLayers = 1024;
constexpr unsigned kMaxGridY = 65535;

// Division of 32-bit unsigned n < 2^31 by a fixed d >= 1: q = (mulhi(m, n) + n) >> l
// with l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1.
struct FastDiv {
    uint32_t d, m, l;
};

static FastDiv make_fastdiv(uint32_t d)
{
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    const uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
    return FastDiv{d, (uint32_t)m, l};
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f)
{
    return (__umulhi(f.m, n) + n) >> f.l;
}

__global__ void __launch_bounds__(kCopyThreads)
k_dasc_pack(const uint8_t *__restrict__ active, int64_t layer_stride, int S_act, int L,
            int n_units, int64_t unit_bytes, FastDiv unit_vecs,
            const int32_t *__restrict__ offsets, const int32_t *__restrict__ unit_index,
            int R_total, const int32_t *__restrict__ src_slot,
            const int32_t *__restrict__ dst_slot, int pair0, uint8_t *__restrict__ packed,
            int S_ckpt, int32_t *__restrict__ err)
{
    __shared__ int32_t offs[kMaxLayers + 1];
    for (int i = threadIdx.x; i <= L; i += kCopyThreads) offs[i] = offsets[i];
    __syncthreads();
    const int n = pair0 + blockIdx.y;
    const int src = src_slot[n], dst = dst_slot[n];
    if (src < 0 || src >= S_act || dst < 0 || dst >= S_ckpt) {
        if (err && threadIdx.x == 0 && blockIdx.x == 0) atomicOr(err, HLA_DEVERR_SLOT);
        return;
    }
    const uint32_t total = (uint32_t)R_total * unit_vecs.d;
    const uint32_t base = blockIdx.x * (kCopyThreads * kCopyVecs) + threadIdx.x;
    const uint8_t *src_base = active + (int64_t)src * n_units * unit_bytes;
    uint8_t *dst_base = packed + (int64_t)dst * R_total * unit_bytes;

    u32x4 buf[kCopyVecs];
    uint8_t *dptr[kCopyVecs];
#pragma unroll
    for (int i = 0; i < kCopyVecs; ++i) {
        const uint32_t e = base + i * kCopyThreads;
        dptr[i] = nullptr;
        if (e >= total) continue;
        const uint32_t p = fdiv(e, unit_vecs);
        const uint32_t off = e - p * unit_vecs.d;
        int lo = 0, hi = L;  // offs[lo] <= p < offs[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if ((uint32_t)offs[mid] <= p) lo = mid; else hi = mid;
        }
        const int u = unit_index[p];
        if (u < 0 || u >= n_units) {
            if (err) atomicOr(err, HLA_DEVERR_PLAN);
            continue;
        }
        const uint8_t *s = src_base + lo * layer_stride + (int64_t)u * unit_bytes + (int64_t)off * 16;
        buf[i] = ld_nt(reinterpret_cast<const u32x4 *>(s));
        dptr[i] = dst_base + (int64_t)p * unit_bytes + (int64_t)off * 16;
    }
#pragma unroll
    for (int i = 0; i < kCopyVecs; ++i)
        if (dptr[i]) st_nt(reinterpret_cast<u32x4 *>(dptr[i]), buf[i]);
}

__global__ void __launch_bounds__(kCopyThreads)
k_dasc_restore(const uint8_t *__restrict__ packed, int S_ckpt, int R_total,
               const int32_t *__restrict__ unit_pos, int L, int n_units, int64_t unit_bytes,
               FastDiv unit_vecs, FastDiv units, const int32_t *__restrict__ src_slot,
               const int32_t *__restrict__ dst_slot, int pair0, uint8_t *__restrict__ active_out,
               int64_t layer_stride, int S_dst, int32_t *__restrict__ err)
{
    const int n = pair0 + blockIdx.y;
    const int src = src_slot[n], dst = dst_slot[n];
    if (src < 0 || src >= S_ckpt || dst < 0 || dst >= S_dst) {
        if (err && threadIdx.x == 0 && blockIdx.x == 0) atomicOr(err, HLA_DEVERR_SLOT);
        return;
    }
    const uint32_t total = (uint32_t)L * (uint32_t)n_units * unit_vecs.d;
    const uint32_t base = blockIdx.x * (kCopyThreads * kCopyVecs) + threadIdx.x;
    const uint8_t *src_base = packed + (int64_t)src * R_total * unit_bytes;
    uint8_t *dst_base = active_out + (int64_t)dst * n_units * unit_bytes;

    u32x4 buf[kCopyVecs];
    uint8_t *dptr[kCopyVecs];
#pragma unroll
    for (int i = 0; i < kCopyVecs; ++i) {
        const uint32_t e = base + i * kCopyThreads;
        dptr[i] = nullptr;
        if (e >= total) continue;
        const uint32_t g = fdiv(e, unit_vecs);   // layer * n_units + unit
        const uint32_t off = e - g * unit_vecs.d;
        const uint32_t l = fdiv(g, units);
        const uint32_t u = g - l * units.d;
        const int pos = unit_pos[g];
        buf[i] = u32x4{0u, 0u, 0u, 0u};
        if (pos >= 0) {
            if (pos < R_total)
                buf[i] = ld_nt(reinterpret_cast<const u32x4 *>(
                    src_base + (int64_t)pos * unit_bytes + (int64_t)off * 16));
            else if (err)
                atomicOr(err, HLA_DEVERR_PLAN);
        }
        dptr[i] = dst_base + (int64_t)l * layer_stride + (int64_t)u * unit_bytes + (int64_t)off * 16;
    }
#pragma unroll
    for (int i = 0; i < kCopyVecs; ++i)
        if (dptr[i]) st_nt(reinterpret_cast<u32x4 *>(dptr[i]), buf[i]);
}

} // namespace hla

extern "C" {

int dasc_pack(const void *active, int64_t layer_stride_bytes, int S_act, int L, int n_units,
              int64_t unit_bytes, const int32_t *offsets, const int32_t *unit_index, int R_total,
              const int32_t *src_slot, const int32_t *dst_slot, int N, void *packed, int S_ckpt,
              int32_t *err_flag, void *stream)
{
    int rc = hla::check_dasc(active, layer_stride_bytes, S_act, L, n_units, unit_bytes, offsets,
                             unit_index, R_total, src_slot, dst_slot, N, packed, S_ckpt);
    if (rc != HLA_OK) return rc;
    if (L > hla::kMaxLayers) return HLA_ERR_UNSUPPORTED;
    if (N == 0 || R_total == 0) return HLA_OK;
    const hla::FastDiv uv = hla::make_fastdiv((uint32_t)(unit_bytes / 16));
    const uint64_t total = (uint64_t)R_total * uv.d;
    const unsigned bx = (unsigned)((total + hla::kCopyThreads * hla::kCopyVecs - 1) /
                                   (hla::kCopyThreads * hla::kCopyVecs));
    hipStream_t st = static_cast<hipStream_t>(stream);
    for (int p0 = 0; p0 < N; p0 += (int)hla::kMaxGridY) {
        const unsigned by = (unsigned)std::min<int>(N - p0, (int)hla::kMaxGridY);
        hipLaunchKernelGGL(hla::k_dasc_pack, dim3(bx, by), dim3(hla::kCopyThreads), 0, st,
                           (const uint8_t *)active, layer_stride_bytes, S_act, L, n_units,
                           unit_bytes, uv, offsets, unit_index, R_total, src_slot, dst_slot, p0,
                           (uint8_t *)packed, S_ckpt, err_flag);
        if (hipGetLastError() != hipSuccess) return HLA_ERR_LAUNCH;
    }
    return HLA_OK;
}

int dasc_restore(const void *packed, int S_ckpt, int R_total, const int32_t *unit_pos, int L,
                 int n_units, int64_t unit_bytes, const int32_t *src_slot,
                 const int32_t *dst_slot, int N, void *active_out, int64_t layer_stride_bytes,
                 int S_dst, int32_t *err_flag, void *stream)
{
    int rc = hla::check_dasc(active_out, layer_stride_bytes, S_dst, L, n_units, unit_bytes,
                             unit_pos, unit_pos, R_total, src_slot, dst_slot, N, packed, S_ckpt);
    if (rc != HLA_OK || N == 0) return rc;
    const hla::FastDiv uv = hla::make_fastdiv((uint32_t)(unit_bytes / 16));
    const hla::FastDiv un = hla::make_fastdiv((uint32_t)n_units);
    const uint64_t total = (uint64_t)L * n_units * uv.d;
    const unsigned bx = (unsigned)((total + hla::kCopyThreads * hla::kCopyVecs - 1) /
                                   (hla::kCopyThreads * hla::kCopyVecs));
    hipStream_t st = static_cast<hipStream_t>(stream);
    for (int p0 = 0; p0 < N; p0 += (int)hla::kMaxGridY) {
        const unsigned by = (unsigned)std::min<int>(N - p0, (int)hla::kMaxGridY);
        hipLaunchKernelGGL(hla::k_dasc_restore, dim3(bx, by), dim3(hla::kCopyThreads), 0, st,
                           (const uint8_t *)packed, S_ckpt, R_total, unit_pos, L, n_units,
                           unit_bytes, uv, un, src_slot, dst_slot, p0, (uint8_t *)active_out,
                           layer_stride_bytes, S_dst, err_flag);
        if (hipGetLastError() != hipSuccess) return HLA_ERR_LAUNCH;
    }
    return HLA_OK;
}

} // extern "C"
