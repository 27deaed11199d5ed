// gfx950 kernels for ragged recurrent-state checkpoints ("dasc: Decay-Aware
// State Compression for Hybrid Linear-Attention Serving", §4.1-§4.2 and
// App. B): pack the retained units of active slots into a flat checkpoint
// buffer, and restore a checkpoint into private slots with the omitted units
// zero-filled.  Both are pure byte movement, so they are written as 16-byte
// vector streams: grid.y = (src, dst) pair, grid.x = chunks of that pair's
// bytes (two or four 16-byte vectors per lane, see below), nontemporal loads
// and stores (each byte is touched once).  The ragged index arithmetic
// (vector -> unit, unit -> layer) uses precomputed magic-number division and
// a binary search over the L+1 layer offsets held in LDS.
//
// The same file holds the INT8-composed checkpoint (App. E.1-E.2: each
// retained key-channel row quantised once at store, dequantised once on a
// hit) and the dasc-wr copy-back of refreshed local units (§4.2).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "hla.h"
#include "hla_codec.h"
#include "hla_device.h"
#include "hla_internal.h"

namespace hla {

constexpr int kCopyThreads = 256;
// 16-byte vectors per lane per block (measured on the checkpoint workloads: the
// restore's copy + zero-fill streams best from 8 KiB blocks, 5.53 -> 5.96 TB/s;
// the pack gains ~1% from them; the copy-back prefers 16 KiB, 5.96 vs 5.71)
constexpr int kPackVecs = 2;
constexpr int kRestoreVecs = 2;
constexpr int kUnitCopyVecs = 4;
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
    const uint32_t base = blockIdx.x * (kCopyThreads * kPackVecs) + threadIdx.x;
    const uint8_t *src_base = active + (int64_t)src * n_units * unit_bytes;
    uint8_t *dst_base = packed + (int64_t)dst * R_total * unit_bytes;

    // three stages, so that no stage waits on a later one's memory (the wave's
    // memory counter is in order): the unit lookups, the loads, the stores
    int unit[kPackVecs];
    uint32_t pv[kPackVecs], offv[kPackVecs];
    int layer[kPackVecs];
#pragma unroll
    for (int i = 0; i < kPackVecs; ++i) {
        const uint32_t e = base + i * kCopyThreads;
        unit[i] = -1;
        if (e >= total) continue;
        pv[i] = fdiv(e, unit_vecs);
        offv[i] = e - pv[i] * unit_vecs.d;
        int lo = 0, hi = L;  // offs[lo] <= p < offs[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if ((uint32_t)offs[mid] <= pv[i]) lo = mid; else hi = mid;
        }
        layer[i] = lo;
        unit[i] = unit_index[pv[i]];
    }
    u32x4 buf[kPackVecs];
    uint8_t *dptr[kPackVecs];
#pragma unroll
    for (int i = 0; i < kPackVecs; ++i) {
        dptr[i] = nullptr;
        if (base + i * kCopyThreads >= total) continue;
        const int u = unit[i];
        if (u < 0 || u >= n_units) {
            if (err) atomicOr(err, HLA_DEVERR_PLAN);
            continue;
        }
        const uint8_t *s = src_base + layer[i] * layer_stride + (int64_t)u * unit_bytes +
                           (int64_t)offv[i] * 16;
        buf[i] = ld_nt(reinterpret_cast<const u32x4 *>(s));
        dptr[i] = dst_base + (int64_t)pv[i] * unit_bytes + (int64_t)offv[i] * 16;
    }
#pragma unroll
    for (int i = 0; i < kPackVecs; ++i)
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
    const uint32_t base = blockIdx.x * (kCopyThreads * kRestoreVecs) + threadIdx.x;
    const uint8_t *src_base = packed + (int64_t)src * R_total * unit_bytes;
    uint8_t *dst_base = active_out + (int64_t)dst * n_units * unit_bytes;

    // three stages, as in k_dasc_pack: lookups (with the destinations), loads, stores
    int pos[kRestoreVecs];
    uint32_t offv[kRestoreVecs];
    uint8_t *dptr[kRestoreVecs];
#pragma unroll
    for (int i = 0; i < kRestoreVecs; ++i) {
        const uint32_t e = base + i * kCopyThreads;
        dptr[i] = nullptr;
        pos[i] = -1;
        if (e >= total) continue;
        const uint32_t g = fdiv(e, unit_vecs);   // layer * n_units + unit
        offv[i] = e - g * unit_vecs.d;
        const uint32_t l = fdiv(g, units);
        const uint32_t u = g - l * units.d;
        pos[i] = unit_pos[g];
        dptr[i] = dst_base + (int64_t)l * layer_stride + (int64_t)u * unit_bytes +
                  (int64_t)offv[i] * 16;
    }
    u32x4 buf[kRestoreVecs];
#pragma unroll
    for (int i = 0; i < kRestoreVecs; ++i) {
        buf[i] = u32x4{0u, 0u, 0u, 0u};
        if (pos[i] >= 0) {
            if (pos[i] < R_total)
                buf[i] = ld_nt(reinterpret_cast<const u32x4 *>(
                    src_base + (int64_t)pos[i] * unit_bytes + (int64_t)offv[i] * 16));
            else if (err)
                atomicOr(err, HLA_DEVERR_PLAN);
        }
    }
#pragma unroll
    for (int i = 0; i < kRestoreVecs; ++i)
        if (dptr[i]) st_nt(reinterpret_cast<u32x4 *>(dptr[i]), buf[i]);
}

// Layer of flat position p: offs[lo] <= p < offs[lo + 1] (offsets in LDS).
__device__ __forceinline__ int layer_of(const int32_t *offs, int L, uint32_t p)
{
    int lo = 0, hi = L;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((uint32_t)offs[mid] <= p) lo = mid; else hi = mid;
    }
    return lo;
}

// ------------------------------------------------------------------ dasc-wr copy-back
//
// Copy the listed units of scratch slot src into active slot dst, layer by
// layer; units not listed are not touched.  The list is a ragged plan of the
// LOCAL units (dasc_plan of the inverted selection mask).
__global__ void __launch_bounds__(kCopyThreads)
k_dasc_copy_units(const uint8_t *__restrict__ scratch, int64_t scratch_stride, int S_scratch,
                  uint8_t *__restrict__ active, int64_t layer_stride, int S_act, int L,
                  int n_units, int64_t unit_bytes, FastDiv unit_vecs,
                  const int32_t *__restrict__ offsets, const int32_t *__restrict__ unit_index,
                  int R_local, const int32_t *__restrict__ src_slot,
                  const int32_t *__restrict__ dst_slot, int pair0, int32_t *__restrict__ err)
{
    __shared__ int32_t offs[kMaxLayers + 1];
    for (int i = threadIdx.x; i <= L; i += kCopyThreads) offs[i] = offsets[i];
    __syncthreads();
    const int n = pair0 + blockIdx.y;
    const int src = src_slot[n], dst = dst_slot[n];
    if (src < 0 || src >= S_scratch || dst < 0 || dst >= S_act) {
        if (err && threadIdx.x == 0 && blockIdx.x == 0) atomicOr(err, HLA_DEVERR_SLOT);
        return;
    }
    const uint32_t total = (uint32_t)R_local * unit_vecs.d;
    const uint32_t base = blockIdx.x * (kCopyThreads * kUnitCopyVecs) + threadIdx.x;
    const uint8_t *src_base = scratch + (int64_t)src * n_units * unit_bytes;
    uint8_t *dst_base = active + (int64_t)dst * n_units * unit_bytes;

    // three stages, as in k_dasc_pack: unit lookups, loads, stores
    int unit[kUnitCopyVecs], layer[kUnitCopyVecs];
    uint32_t offv[kUnitCopyVecs];
#pragma unroll
    for (int i = 0; i < kUnitCopyVecs; ++i) {
        const uint32_t e = base + i * kCopyThreads;
        unit[i] = -1;
        if (e >= total) continue;
        const uint32_t p = fdiv(e, unit_vecs);
        offv[i] = e - p * unit_vecs.d;
        layer[i] = layer_of(offs, L, p);
        unit[i] = unit_index[p];
    }
    u32x4 buf[kUnitCopyVecs];
    uint8_t *dptr[kUnitCopyVecs];
#pragma unroll
    for (int i = 0; i < kUnitCopyVecs; ++i) {
        dptr[i] = nullptr;
        if (base + i * kCopyThreads >= total) continue;
        const int u = unit[i];
        if (u < 0 || u >= n_units) {
            if (err) atomicOr(err, HLA_DEVERR_PLAN);
            continue;
        }
        const int64_t unit_off = (int64_t)u * unit_bytes + (int64_t)offv[i] * 16;
        buf[i] = ld_nt(reinterpret_cast<const u32x4 *>(src_base + layer[i] * scratch_stride +
                                                        unit_off));
        dptr[i] = dst_base + layer[i] * layer_stride + unit_off;
    }
#pragma unroll
    for (int i = 0; i < kUnitCopyVecs; ++i)
        if (dptr[i]) st_nt(reinterpret_cast<u32x4 *>(dptr[i]), buf[i]);
}

// ------------------------------------------------------------------ INT8 checkpoints
//
// One FP32 row of dv values is handled by CG = dv/8 adjacent lanes, 8 values
// per lane: values 4*cg .. 4*cg+3 of each half of the row, so that every
// 16-byte FP32 access and every 4-byte code access of a wave is contiguous
// across the row's lanes (whole 64-byte segments per instruction).  A block
// of 256 threads covers 256/CG rows per pass and a few passes, with
// every pass's loads issued before the first conversion.  The row maximum is a DPP max over the
// CG lanes; codes and scale come from the shared codec (hla_codec.h).
// passes per block, measured on the checkpoint workloads: pack 4; restore 2
// for one-row units (KDA channel rows: 4.84 -> 5.49 TB/s), 1 for larger units
// (GDN heads: 5.90 TB/s at 1, 5.44 at 2; more passes were slower for both)
constexpr int kInt8PassesPack = 4;
inline int int8_restore_passes(int unit_rows) { return unit_rows == 1 ? 2 : 1; }

template <int DV>
__global__ void __launch_bounds__(kCopyThreads)
k_dasc_pack_int8(const uint8_t *__restrict__ active, int64_t layer_stride, int S_act, int L,
                 int n_units, int log2_rows, const int32_t *__restrict__ offsets,
                 const int32_t *__restrict__ unit_index, int R_total,
                 const int32_t *__restrict__ src_slot, const int32_t *__restrict__ dst_slot,
                 int pair0, int8_t *__restrict__ codes, float *__restrict__ scales, int S_ckpt,
                 int32_t *__restrict__ err)
{
    constexpr int CG = DV / 8, LCG = Log2<CG>::v, RPP = kCopyThreads / CG;
    __shared__ int32_t offs[kMaxLayers + 1];
    for (int i = threadIdx.x; i <= L; i += kCopyThreads) offs[i] = offsets[i];
    __syncthreads();
    const int n = pair0 + blockIdx.y;
    const int src = src_slot[n], dst = dst_slot[n];
    if (src < 0 || src >= S_act || dst < 0 || dst >= S_ckpt) {
        if (err && threadIdx.x == 0 && blockIdx.x == 0) atomicOr(err, HLA_DEVERR_SLOT);
        return;
    }
    const int cg = threadIdx.x & (CG - 1);
    const uint32_t rows = (uint32_t)R_total << log2_rows;
    const uint32_t row_mask = (1u << log2_rows) - 1u;
    const uint8_t *src_base = active + (int64_t)src * n_units * ((int64_t)DV * 4 << log2_rows);
    // three stages, so that no stage waits on a later one's memory (the wave's
    // memory counter is in order): unit lookups, row loads, quantise + stores
    constexpr int P = kInt8PassesPack;
    bool live[P], skip[P];
    int unit[P], layer[P];
    uint32_t rrv[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        rrv[i] = (blockIdx.x * P + i) * RPP + (threadIdx.x >> LCG);
        live[i] = rrv[i] < rows;  // uniform over a row's CG lanes
        unit[i] = 0;
        layer[i] = 0;
        if (!live[i]) continue;
        const uint32_t p = rrv[i] >> log2_rows;
        layer[i] = layer_of(offs, L, p);
        unit[i] = unit_index[p];
    }
    float x[P][8];
    uint32_t out_row[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        out_row[i] = 0;
        skip[i] = false;
        if (!live[i]) continue;
        const uint32_t r = rrv[i] & row_mask;
        int u = unit[i];
        if (u < 0 || u >= n_units) {
            // the row's lanes still load (unit 0) and exchange their maximum together;
            // nothing is stored for it, and the flag reports the plan
            if (err) atomicOr(err, HLA_DEVERR_PLAN);
            u = 0;
            skip[i] = true;
        }
        const float *row = reinterpret_cast<const float *>(
            src_base + layer[i] * layer_stride + ((((int64_t)u << log2_rows) + r) * DV) * 4);
        const f32x4 a = ld_nt(reinterpret_cast<const f32x4 *>(row + cg * 4));
        const f32x4 b = ld_nt(reinterpret_cast<const f32x4 *>(row + DV / 2 + cg * 4));
        x[i][0] = a.x; x[i][1] = a.y; x[i][2] = a.z; x[i][3] = a.w;
        x[i][4] = b.x; x[i][5] = b.y; x[i][6] = b.z; x[i][7] = b.w;
        out_row[i] = ((uint32_t)dst * (uint32_t)R_total << log2_rows) + rrv[i];
    }
#pragma unroll
    for (int i = 0; i < kInt8PassesPack; ++i) {
        if (!live[i]) continue;
        const float amax = max_low_lane_bits<LCG>(row_absmax8(x[i]));
        uint32_t w0, w1;
        const float s = encode_int8(x[i], amax, w0, w1);
        if (skip[i]) continue;
        int8_t *crow = codes + (int64_t)out_row[i] * DV;
        st_nt(reinterpret_cast<uint32_t *>(crow + cg * 4), w0);
        st_nt(reinterpret_cast<uint32_t *>(crow + DV / 2 + cg * 4), w1);
        if (cg == 0) scales[out_row[i]] = s;
    }
}

template <int DV, int P>
__global__ void __launch_bounds__(kCopyThreads)
k_dasc_restore_int8(const int8_t *__restrict__ codes, const float *__restrict__ scales,
                    int S_ckpt, int R_total, const int32_t *__restrict__ unit_pos, int L,
                    int n_units, FastDiv units, int log2_rows,
                    const int32_t *__restrict__ src_slot, const int32_t *__restrict__ dst_slot,
                    int pair0, uint8_t *__restrict__ active_out, int64_t layer_stride,
                    int S_dst, int32_t *__restrict__ err)
{
    constexpr int CG = DV / 8, LCG = Log2<CG>::v, RPP = kCopyThreads / CG;
    const int n = pair0 + blockIdx.y;
    const int src = src_slot[n], dst = dst_slot[n];
    if (src < 0 || src >= S_ckpt || dst < 0 || dst >= S_dst) {
        if (err && threadIdx.x == 0 && blockIdx.x == 0) atomicOr(err, HLA_DEVERR_SLOT);
        return;
    }
    const int cg = threadIdx.x & (CG - 1);
    const uint32_t rows = ((uint32_t)L * (uint32_t)n_units) << log2_rows;
    const uint32_t row_mask = (1u << log2_rows) - 1u;
    uint8_t *dst_base = active_out + (int64_t)dst * n_units * ((int64_t)DV * 4 << log2_rows);
    // Three stages over the lane's P rows, so that no stage waits on a later
    // one's memory: every unit_pos lookup (with the destination addresses),
    // then every code / scale load, then the stores (a lookup issued after a
    // row's code loads could only be used once those loads had returned too).
    int pos[P];
    uint32_t rr[P];
    bool live[P];
    float *d[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        rr[i] = (blockIdx.x * P + i) * RPP + (threadIdx.x >> LCG);
        live[i] = rr[i] < rows;  // uniform over a row's CG lanes
        const uint32_t g = rr[i] >> log2_rows, r = rr[i] & row_mask;  // g = l * n_units + u
        pos[i] = live[i] ? unit_pos[g] : -1;
        const uint32_t l = fdiv(g, units);
        const uint32_t u = g - l * units.d;
        d[i] = reinterpret_cast<float *>(dst_base + l * layer_stride +
                                         ((((int64_t)u << log2_rows) + r) * DV) * 4) + cg * 4;
    }
    uint32_t w0[P], w1[P];
    float sc[P];
    // With one row per lane (head units: a workgroup's rows share one unit) an
    // omitted row's zeros go out right behind its lookup, ahead of any load:
    // 5.88 -> 6.1 TB/s on the GDN checkpoint workload.  With two rows per lane
    // (channel-row units, a wave mixing omitted and retained rows) the same order
    // measured 12% slower, a wave's zero stores delaying its loads, so there the
    // zeros stay in the last stage.
    constexpr bool zeros_first = P == 1;
    if constexpr (zeros_first) {
        if (live[0] && pos[0] < 0) {
            st_nt(reinterpret_cast<f32x4 *>(d[0]), f32x4{0.0f, 0.0f, 0.0f, 0.0f});
            st_nt(reinterpret_cast<f32x4 *>(d[0] + DV / 2), f32x4{0.0f, 0.0f, 0.0f, 0.0f});
        }
    }
#pragma unroll
    for (int i = 0; i < P; ++i) {
        w0[i] = w1[i] = 0u;
        sc[i] = 0.0f;
        if (pos[i] >= 0) {
            if (pos[i] < R_total) {
                const int64_t in_row =
                    (((int64_t)src * R_total + pos[i]) << log2_rows) + (rr[i] & row_mask);
                const int8_t *crow = codes + in_row * DV;
                w0[i] = ld_nt(reinterpret_cast<const uint32_t *>(crow + cg * 4));
                w1[i] = ld_nt(reinterpret_cast<const uint32_t *>(crow + DV / 2 + cg * 4));
                sc[i] = scales[in_row];
            } else if (err) {
                atomicOr(err, HLA_DEVERR_PLAN);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < P; ++i) {
        if (!live[i] || (zeros_first && pos[i] < 0)) continue;
        float y[8];
        decode_int8(w0[i], w1[i], sc[i], y);  // q * s, one FP32 rounding (0 when omitted)
        st_nt(reinterpret_cast<f32x4 *>(d[i]), f32x4{y[0], y[1], y[2], y[3]});
        st_nt(reinterpret_cast<f32x4 *>(d[i] + DV / 2), f32x4{y[4], y[5], y[6], y[7]});
    }
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
    if (rc == HLA_OK && N > 0)
        rc = hla::check_dasc_tables(
            hla::Range{packed, (size_t)((int64_t)S_ckpt * R_total * unit_bytes)}, hla::Range{},
            offsets, L, unit_index, R_total, nullptr, 0, src_slot, dst_slot, N);
    if (rc != HLA_OK) return rc;
    if (L > hla::kMaxLayers) return HLA_ERR_UNSUPPORTED;
    if (N == 0 || R_total == 0) return HLA_OK;
    const hla::FastDiv uv = hla::make_fastdiv((uint32_t)(unit_bytes / 16));
    const uint64_t total = (uint64_t)R_total * uv.d;
    const unsigned bx = (unsigned)((total + hla::kCopyThreads * hla::kPackVecs - 1) /
                                   (hla::kCopyThreads * hla::kPackVecs));
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
    if (rc == HLA_OK && N > 0)
        rc = hla::check_dasc_tables(
            hla::Range{active_out,
                       (size_t)hla::dasc_span(layer_stride_bytes, L, S_dst, n_units, unit_bytes)},
            hla::Range{}, nullptr, L, nullptr, 0, unit_pos, n_units, src_slot, dst_slot, N);
    if (rc != HLA_OK || N == 0) return rc;
    const hla::FastDiv uv = hla::make_fastdiv((uint32_t)(unit_bytes / 16));
    const hla::FastDiv un = hla::make_fastdiv((uint32_t)n_units);
    const uint64_t total = (uint64_t)L * n_units * uv.d;
    const unsigned bx = (unsigned)((total + hla::kCopyThreads * hla::kRestoreVecs - 1) /
                                   (hla::kCopyThreads * hla::kRestoreVecs));
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

int dasc_refresh_local(const void *scratch, int64_t scratch_layer_stride_bytes, int S_scratch,
                       void *active, int64_t layer_stride_bytes, int S_act, int L, int n_units,
                       int64_t unit_bytes, const int32_t *offsets, const int32_t *unit_index,
                       int R_local, const int32_t *src_slot, const int32_t *dst_slot, int N,
                       int32_t *err_flag, void *stream)
{
    // the scratch side as the "packed" operand only for the alias test; its own
    // geometry is checked as a second active-style layout
    int rc = hla::check_dasc(active, layer_stride_bytes, S_act, L, n_units, unit_bytes, offsets,
                             unit_index, R_local, src_slot, dst_slot, N, scratch, 0);
    if (rc == HLA_OK)
        rc = hla::check_dasc(scratch, scratch_layer_stride_bytes, S_scratch, L, n_units,
                             unit_bytes, offsets, unit_index, R_local, src_slot, dst_slot, N,
                             active, 0);
    if (rc == HLA_OK && N > 0 && scratch && active) {
        const int64_t span_a = (L - 1) * layer_stride_bytes + (int64_t)S_act * n_units * unit_bytes;
        const int64_t span_s =
            (L - 1) * scratch_layer_stride_bytes + (int64_t)S_scratch * n_units * unit_bytes;
        if (hla::overlaps(hla::Range{active, (size_t)span_a}, hla::Range{scratch, (size_t)span_s}))
            rc = HLA_ERR_ALIAS;
        if (rc == HLA_OK)
            rc = hla::check_dasc_tables(hla::Range{active, (size_t)span_a}, hla::Range{},
                                        offsets, L, unit_index, R_local, nullptr, 0, src_slot,
                                        dst_slot, N);
    }
    if (rc != HLA_OK) return rc;
    if (L > hla::kMaxLayers) return HLA_ERR_UNSUPPORTED;
    if (N == 0 || R_local == 0) return HLA_OK;
    const hla::FastDiv uv = hla::make_fastdiv((uint32_t)(unit_bytes / 16));
    const uint64_t total = (uint64_t)R_local * uv.d;
    const unsigned bx = (unsigned)((total + hla::kCopyThreads * hla::kUnitCopyVecs - 1) /
                                   (hla::kCopyThreads * hla::kUnitCopyVecs));
    hipStream_t st = static_cast<hipStream_t>(stream);
    for (int p0 = 0; p0 < N; p0 += (int)hla::kMaxGridY) {
        const unsigned by = (unsigned)std::min<int>(N - p0, (int)hla::kMaxGridY);
        hipLaunchKernelGGL(hla::k_dasc_copy_units, dim3(bx, by), dim3(hla::kCopyThreads), 0, st,
                           (const uint8_t *)scratch, scratch_layer_stride_bytes, S_scratch,
                           (uint8_t *)active, layer_stride_bytes, S_act, L, n_units, unit_bytes,
                           uv, offsets, unit_index, R_local, src_slot, dst_slot, p0, err_flag);
        if (hipGetLastError() != hipSuccess) return HLA_ERR_LAUNCH;
    }
    return HLA_OK;
}

int dasc_pack_int8(const float *active, int64_t layer_stride_bytes, int S_act, int L, int n_units,
                   int unit_rows, int dv, const int32_t *offsets, const int32_t *unit_index,
                   int R_total, const int32_t *src_slot, const int32_t *dst_slot, int N,
                   int8_t *codes, float *scales, int S_ckpt, int32_t *err_flag, void *stream)
{
    int rc = hla::check_dasc_int8(active, layer_stride_bytes, S_act, L, n_units, unit_rows, dv,
                                  offsets, unit_index, R_total, src_slot, dst_slot, N, codes,
                                  scales, S_ckpt);
    if (rc == HLA_OK && N > 0) {
        const size_t rows = (size_t)S_ckpt * R_total * unit_rows;
        rc = hla::check_dasc_tables(hla::Range{codes, rows * dv},
                                    hla::Range{scales, rows * sizeof(float)}, offsets, L,
                                    unit_index, R_total, nullptr, 0, src_slot, dst_slot, N);
    }
    if (rc != HLA_OK) return rc;
    if (L > hla::kMaxLayers) return HLA_ERR_UNSUPPORTED;
    if (N == 0 || R_total == 0) return HLA_OK;
    const int lr = hla::log2_exact(unit_rows);
    const uint64_t rows = (uint64_t)R_total << lr;
    const uint64_t per_block = (uint64_t)(hla::kCopyThreads / (dv / 8)) * hla::kInt8PassesPack;
    const unsigned bx = (unsigned)((rows + per_block - 1) / per_block);
    hipStream_t st = static_cast<hipStream_t>(stream);
    for (int p0 = 0; p0 < N; p0 += (int)hla::kMaxGridY) {
        const unsigned by = (unsigned)std::min<int>(N - p0, (int)hla::kMaxGridY);
        const dim3 grid(bx, by), block(hla::kCopyThreads);
        if (dv == 128)
            hipLaunchKernelGGL(hla::k_dasc_pack_int8<128>, grid, block, 0, st,
                               (const uint8_t *)active, layer_stride_bytes, S_act, L, n_units, lr,
                               offsets, unit_index, R_total, src_slot, dst_slot, p0, codes,
                               scales, S_ckpt, err_flag);
        else
            hipLaunchKernelGGL(hla::k_dasc_pack_int8<64>, grid, block, 0, st,
                               (const uint8_t *)active, layer_stride_bytes, S_act, L, n_units, lr,
                               offsets, unit_index, R_total, src_slot, dst_slot, p0, codes,
                               scales, S_ckpt, err_flag);
        if (hipGetLastError() != hipSuccess) return HLA_ERR_LAUNCH;
    }
    return HLA_OK;
}

int dasc_restore_int8(const int8_t *codes, const float *scales, int S_ckpt, int R_total,
                      const int32_t *unit_pos, int L, int n_units, int unit_rows, int dv,
                      const int32_t *src_slot, const int32_t *dst_slot, int N, float *active_out,
                      int64_t layer_stride_bytes, int S_dst, int32_t *err_flag, void *stream)
{
    int rc = hla::check_dasc_int8(active_out, layer_stride_bytes, S_dst, L, n_units, unit_rows,
                                  dv, unit_pos, unit_pos, R_total, src_slot, dst_slot, N, codes,
                                  scales, S_ckpt);
    if (rc == HLA_OK && N > 0)
        rc = hla::check_dasc_tables(
            hla::Range{active_out, (size_t)hla::dasc_span(layer_stride_bytes, L, S_dst, n_units,
                                                          (int64_t)unit_rows * dv * 4)},
            hla::Range{}, nullptr, L, nullptr, 0, unit_pos, n_units, src_slot, dst_slot, N);
    if (rc != HLA_OK || N == 0) return rc;
    // units of 2-8 rows with at most half of them retained: by blocks of 128 rows
    // (measured 5-13% faster there, checkpoints read cold; see restore_int8_by_blocks)
    if (unit_rows >= 2 && unit_rows <= 8 && (int64_t)R_total * 2 <= (int64_t)L * n_units &&
        hla::restore_int8_by_blocks(codes, scales, S_ckpt, R_total, unit_pos, L, n_units,
                                    unit_rows, dv, src_slot, dst_slot, N, active_out,
                                    layer_stride_bytes, S_dst, err_flag, stream))
        return hipGetLastError() == hipSuccess ? HLA_OK : HLA_ERR_LAUNCH;
    const int lr = hla::log2_exact(unit_rows);
    const hla::FastDiv un = hla::make_fastdiv((uint32_t)n_units);
    const uint64_t rows = ((uint64_t)L * n_units) << lr;
    const int passes = hla::int8_restore_passes(unit_rows);
    const uint64_t per_block = (uint64_t)(hla::kCopyThreads / (dv / 8)) * passes;
    const unsigned bx = (unsigned)((rows + per_block - 1) / per_block);
    hipStream_t st = static_cast<hipStream_t>(stream);
    for (int p0 = 0; p0 < N; p0 += (int)hla::kMaxGridY) {
        const unsigned by = (unsigned)std::min<int>(N - p0, (int)hla::kMaxGridY);
        const dim3 grid(bx, by), block(hla::kCopyThreads);
#define HLA_RESTORE8(DV_, P_)                                                                 \
    hipLaunchKernelGGL((hla::k_dasc_restore_int8<DV_, P_>), grid, block, 0, st, codes, scales,  \
                       S_ckpt, R_total, unit_pos, L, n_units, un, lr, src_slot, dst_slot, p0,  \
                       (uint8_t *)active_out, layer_stride_bytes, S_dst, err_flag)
        if (dv == 128) {
            if (passes == 2) HLA_RESTORE8(128, 2); else HLA_RESTORE8(128, 1);
        } else {
            if (passes == 2) HLA_RESTORE8(64, 2); else HLA_RESTORE8(64, 1);
        }
#undef HLA_RESTORE8
        if (hipGetLastError() != hipSuccess) return HLA_ERR_LAUNCH;
    }
    return HLA_OK;
}

} // extern "C"
