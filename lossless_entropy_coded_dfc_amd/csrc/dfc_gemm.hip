// dfc_gemm.hip - fused decode + matrix product Y = W X on gfx950, for W
// stored as a panel-layout DFC1 container (bf16 weights whose exponents are
// Huffman-coded, DFloat11 blog, sections 02 and 03).
//
// The weights are decoded exactly as by the flat decoder (count pass,
// wavefront scan, write pass into LDS), but the decoded values never reach
// HBM: each complete 32 x 16 sub-tile of W is assembled from its staged
// exponents and raw bytes straight into the A operand of one 32x32x16 bf16
// MFMA per 32 output columns, and the products accumulate in fp32 registers.
//
// Work decomposition: a workgroup takes whole panels (32 rows of W), a few
// wavefronts per panel, or, for matrices with too few panels to fill the
// GPU, a share of one panel's items; each wavefront decodes some items (32
// rows x panel_k columns) and accumulates their products in registers.
// A block of an item (64 chunks) decodes into the wavefront's staging area,
// whose start is the first sub-tile the block touches; the exponents of a
// sub-tile the block only begins are carried in registers into the next
// block's staging area.  The partial 32 x B products of a panel's wavefronts
// are then summed in LDS in wavefront order and written to Y with plain
// stores: no atomics, and the same bits on every run.  Only when a panel is
// shared by several workgroups are their sums added into Y (zeroed first)
// with fp32 atomics.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>

#include "dfc.h"
#include "dfc_decode_core.h"
#include "dfc_format.h"

namespace {

using bf16x8 = __attribute__((ext_vector_type(8))) __bf16;
using f32x16 = __attribute__((ext_vector_type(16))) float;

struct GemmArgs {
    const uint32_t *words;     // code stream (with its guard words)
    const uint32_t *offw;      // packed 5-bit chunk offsets
    const uint32_t *blockout;  // u32 out[n_blocks + 1], indices in panel order
    const uint32_t *items;     // (n_items + 1) x {first chunk, first block, code bits, 0}
    const uint8_t *raw;        // raw bytes in panel order
    const uint8_t *tables;     // derived decode tables
    const uint16_t *x;         // B vectors of K bf16: x[b K + k]
    float *y;                  // B vectors of M fp32: y[b M + m]
    uint32_t words_bytes, offw_bytes, raw_bytes, x_bytes, y_bytes;
    uint32_t n_panels, slices, panel_k, cols, rows, batch;
    uint32_t wpp, group;       // wavefronts per panel in a workgroup, panels per workgroup
    uint32_t split, rounds;    // workgroups per panel; rounds = ceil(n_panels / group) * split
    uint32_t tables_bytes, lut_bits, stage_bytes;
    uint32_t *status;
};

// Sub-tiles (512 values) whose raw bytes are prefetched into registers per
// block: a 64-chunk block of about 3 bits per code completes at most this
// many; the rest load when used.
template <int C>
struct GemmPrefetch {
    static constexpr int N = C >= 32 ? 10 : (C == 16 ? 8 : (C == 8 ? 4 : 3));
};

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &v) { return __builtin_bit_cast(bf16x8, v); }

// One item (32 rows x panel_k columns of W, item q of the container): its
// blocks are decoded and each complete sub-tile is multiplied into acc.
// Returns false (and sets the status word) if a block's decoded count
// disagrees with its block offsets; acc then holds a partial sum.
template <int C, int NT>
__device__ __forceinline__ bool gemm_item(const GemmArgs &g, uint32_t q, const Tables &t, uint8_t *stage,
                                          uint32_t stage_off, uint32_t lane, const __amdgpu_buffer_rsrc_t &words,
                                          const __amdgpu_buffer_rsrc_t &offw, const __amdgpu_buffer_rsrc_t &raw,
                                          const __amdgpu_buffer_rsrc_t &xr, uint32_t xcol, f32x16 (&acc)[NT]) {
    constexpr int PF = GemmPrefetch<C>::N;
    extern __shared__ __align__(16) uint8_t lds[];
    const const_u32_ptr items = (const_u32_ptr)(g.items);
    const const_u32_ptr blockout = (const_u32_ptr)(g.blockout);
    const uint32_t c0 = items[4 * q], b0 = items[4 * q + 1], bits = items[4 * q + 2];
    const uint32_t b1 = items[4 * q + 5];
    const uint32_t p = q / g.slices, col0 = (q % g.slices) * g.panel_k;
    const uint32_t e0 = 32u * (p * g.cols + col0);
    u32x2 carry = {0u, 0u};
    for (uint32_t b = b0; b < b1; ++b) {
        const uint32_t s_out = blockout[b], e_out = blockout[b + 1];
        const uint32_t rs = s_out - e0, base = rs & ~511u, lead = rs - base;
        const uint32_t total_want = e_out - s_out;
        // Zero the staging bytes this block ORs into, then put back the
        // exponents carried from the previous block in front of them.
        const uint32_t nz = min(lead + total_want + 8u, g.stage_bytes);
        for (uint32_t o = 16u * lane; o + 16u <= ((nz + 15u) & ~15u); o += 16u * kWave)
            *reinterpret_cast<uint4 *>(stage + o) = make_uint4(0, 0, 0, 0);
        if (8u * lane < lead) *reinterpret_cast<u32x2 *>(stage + 8u * lane) = carry;

        const uint32_t ci = (b - b0) * kWave + lane;  // item-relative chunk
        Chunk<C> ck;
        load_chunk<C>(words, offw, c0 + ci, ck);
        // raw bytes only for the sub-tiles this block completes: the one it
        // only begins is carried as exponents, and the next block loads its
        // raw bytes
        const uint32_t rounds = (lead + total_want) >> 9;
        u32x2 R[PF];
#pragma unroll
        for (int j = 0; j < PF; ++j)
            R[j] = uint32_t(j) < rounds ? __builtin_amdgcn_raw_buffer_load_b64(raw, e0 + base + 512u * j + 8u * lane, 0, 0)
                                        : u32x2{0u, 0u};
        int start, end;
        chunk_span<C>(ck, c0 + ci,
                      int(min(max(int64_t(bits) - int64_t(ci) * (8 * C), int64_t(-1)), int64_t(8 * C + 32))),
                      start, end);
        // count and write passes at a raised wave priority, the products at the
        // normal one (wavefronts that are decoding issue first; 1-3% in
        // one-process timing)
        __builtin_amdgcn_s_setprio(1);
        const uint32_t cnt = start < end ? count_codes<C>(ck, start, end, t) : 0u;
        const uint32_t incl = wave_inclusive_scan(cnt);
        const uint32_t total = __builtin_amdgcn_readlane(incl, kWave - 1);
        const bool bad = (total != total_want) | (__builtin_amdgcn_ballot_w64(cnt > 8u * C) != 0);
        if (!bad && cnt) write_codes<C>(ck, start, end, lds, stage_off + lead + (incl - cnt), t);
        wait_for(R);
        if (bad) {
            if (lane == 0 && g.status) atomicOr(g.status, kStatusCorrupt);
            return false;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        __builtin_amdgcn_s_setprio(0);
        // Complete sub-tiles: W operand from the staged exponents and the
        // raw bytes, X operand from global memory (cached); the X fragments of
        // all column tiles are requested before their products, so that their
        // cache round trips overlap (1-2% at 64 columns).
        const uint32_t extent = lead + total;
        const uint32_t nfull = extent >> 9;
        const uint32_t kcol = col0 + 16u * (base >> 9);
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            if (uint32_t(j) < nfull) {
                const u32x2 E = *reinterpret_cast<const u32x2 *>(stage + 512u * j + 8u * lane);
                const bf16x8 A = as_bf16x8(assemble8(E, R[j]));
                u32x4 X[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    X[nt] = __builtin_amdgcn_raw_buffer_load_b128(xr, xcol + 2u * (32u * nt * g.cols + kcol + 16u * j), 0, 0);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, as_bf16x8(X[nt]), acc[nt], 0, 0, 0);
            }
        }
        for (uint32_t j = PF; j < nfull; ++j) {
            const u32x2 Rj = __builtin_amdgcn_raw_buffer_load_b64(raw, e0 + base + 512u * j + 8u * lane, 0, 0);
            const u32x2 E = *reinterpret_cast<const u32x2 *>(stage + 512u * j + 8u * lane);
            const bf16x8 A = as_bf16x8(assemble8(E, Rj));
            u32x4 X[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                X[nt] = __builtin_amdgcn_raw_buffer_load_b128(xr, xcol + 2u * (32u * nt * g.cols + kcol + 16u * j), 0, 0);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, as_bf16x8(X[nt]), acc[nt], 0, 0, 0);
        }
        // The sub-tile this block only began moves to the next block.
        const uint32_t tail = extent - 512u * nfull;
        carry = 8u * lane < tail ? *reinterpret_cast<const u32x2 *>(stage + 512u * nfull + 8u * lane) : u32x2{0u, 0u};
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    return true;
}

// Workgroup of group x wpp wavefronts.  A round takes `group` consecutive
// panels (split == 1) or the part-th of split workgroups on one panel
// (group == 1); a panel's split * wpp wavefronts take its slices in turn:
// wavefront v of the panel takes slices v, v + split wpp, ...  Every staging
// area holds at least 4 KB, which the reduction reuses for one 32 x 32 fp32
// tile per wavefront.
template <int C, int NT>
__global__ __launch_bounds__(1024) void dfc_gemm_kernel(const GemmArgs g) {
    extern __shared__ __align__(16) uint8_t lds[];
    const Tables t = stage_tables(lds, g.tables, g.tables_bytes, g.lut_bits);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t lane = threadIdx.x % kWave;
    const uint32_t wpp = g.wpp;
    const uint32_t pw = wave / wpp, sw = wave % wpp;  // panel in the round, first slice
    const uint32_t stage_off = g.tables_bytes + wave * g.stage_bytes;
    uint8_t *stage = lds + stage_off;
    const __amdgpu_buffer_rsrc_t words =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t *>(g.words), 0, int(g.words_bytes), kBufferConfig);
    const __amdgpu_buffer_rsrc_t offw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t *>(g.offw), 0, int(g.offw_bytes), kBufferConfig);
    const __amdgpu_buffer_rsrc_t raw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(g.raw), 0, int(g.raw_bytes), kBufferConfig);
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(g.x), 0, int(g.x_bytes), kBufferConfig);
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(g.y, 0, int(g.y_bytes), kBufferConfig);
    // B operand rows of this lane: column n = 32 nt + lane % 32 of X, k offset
    // 8 (lane / 32) inside the sub-tile (rows past B load zeros).
    const uint32_t xcol = 2u * (lane % 32u) * g.cols + 16u * (lane / 32u);

    const uint32_t stride = g.split * wpp;
    // the round count is the same for every wavefront of the workgroup
    for (uint32_t r = blockIdx.x; r < g.rounds; r += gridDim.x) {
        const uint32_t part = r % g.split;
        const uint32_t p = (r / g.split) * g.group + pw;
        f32x16 acc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x16{};
        if (p < g.n_panels)
            for (uint32_t s = part * wpp + sw; s < g.slices; s += stride)
                if (!gemm_item<C, NT>(g, p * g.slices + s, t, stage, stage_off, lane, words, offw, raw, xr, xcol, acc))
                    break;
        // D[i][j] of a 32x32 tile: i = 8 (r / 4) + 4 (lane / 32) + r % 4,
        // j = lane % 32.  Value r of lane L goes to slot 4 (64 (r / 4) + L) +
        // r % 4 of the wavefront's tile, so that element e of a float4 slot
        // holds rows 8 (e / 64) + 4 ((e % 64) / 32) + 0..3 of column e % 32.
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            if (nt > 0) __syncthreads();  // the previous tile has been read
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
                *reinterpret_cast<float4 *>(stage + 16u * (64u * r4 + lane)) =
                    make_float4(acc[nt][4 * r4], acc[nt][4 * r4 + 1], acc[nt][4 * r4 + 2], acc[nt][4 * r4 + 3]);
            __syncthreads();
            for (uint32_t e = sw * kWave + lane; e < 256u; e += wpp * kWave) {
                const uint8_t *slot = lds + g.tables_bytes + pw * wpp * g.stage_bytes + 16u * e;
                float4 v = *reinterpret_cast<const float4 *>(slot);
                for (uint32_t w = 1; w < wpp; ++w) {
                    const float4 u = *reinterpret_cast<const float4 *>(slot + w * g.stage_bytes);
                    v.x += u.x;
                    v.y += u.y;
                    v.z += u.z;
                    v.w += u.w;
                }
                const uint32_t n = 32u * uint32_t(nt) + e % 32u;
                const uint32_t m = 32u * p + 8u * (e / 64u) + 4u * ((e % 64u) / 32u);
                if (p < g.n_panels && n < g.batch) {
                    if (g.split == 1) {
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), yr, 4u * (n * g.rows + m), 0, 0);
                    } else {
                        float *yp = g.y + (uint64_t(n) * g.rows + m);
                        unsafeAtomicAdd(yp, v.x);
                        unsafeAtomicAdd(yp + 1, v.y);
                        unsafeAtomicAdd(yp + 2, v.z);
                        unsafeAtomicAdd(yp + 3, v.w);
                    }
                }
            }
        }
        __syncthreads();  // tiles read before the next round's staging
    }
}

__global__ void fill_zero_kernel(float *y, uint64_t n) {
    for (uint64_t i = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += uint64_t(gridDim.x) * blockDim.x)
        y[i] = 0.0f;
}

template <int C, int NT>
dfc_status launch_gemm(const GemmArgs &proto, uint32_t max_block, hipStream_t stream) {
    GemmArgs g = proto;
    // staging: a carried partial sub-tile (< 512) + the block + spill, rounded
    // to 16, and at least one 32 x 32 fp32 tile for the reduction
    const uint32_t stage = std::max(4096u, (511u + max_block + 32u + 15u) & ~15u);
    g.stage_bytes = stage;
    if (!allow_full_lds(reinterpret_cast<const void *>(&dfc_gemm_kernel<C, NT>))) return DFC_EHIP;
    // about 8 wavefronts per workgroup: up to 8 per panel (one slice each
    // when the panel has 8 slices or fewer), several panels when it has few
    uint32_t wpp = std::min<uint32_t>(g.slices, 8u);
    uint32_t group = std::max<uint32_t>(1u, 8u / wpp);
    while (wpp * group > 1 && g.tables_bytes + wpp * group * stage > kLdsBytes) {
        if (group > 1)
            --group;
        else
            --wpp;
    }
    const uint32_t waves = wpp * group;
    const size_t lds = size_t(g.tables_bytes) + size_t(waves) * stage;
    if (lds > kLdsBytes) return DFC_EUNSUPPORTED;
    // Too few panels for the resident wavefronts: share each panel among
    // `split` workgroups, with as few slices per wavefront as the resident
    // count allows, spread evenly.
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(&dfc_gemm_kernel<C, NT>),
                                                     int(waves * kWave), lds) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    const uint64_t resident = uint64_t(per_cu) * waves * uint64_t(device_cu_count());
    uint32_t split = 1;
    if (group == 1 && uint64_t(g.n_panels) * wpp < resident && g.slices > wpp) {
        const uint64_t want = std::min<uint64_t>(g.slices, dfc::ceil_div(resident, uint64_t(g.n_panels)));
        const uint64_t per_wave = dfc::ceil_div(uint64_t(g.slices), want);
        const uint64_t per_panel = dfc::ceil_div(uint64_t(g.slices), per_wave);
        split = uint32_t(dfc::ceil_div(per_panel, uint64_t(wpp)));
    }
    g.wpp = wpp;
    g.group = group;
    g.split = split;
    const uint64_t rounds = dfc::ceil_div(uint64_t(g.n_panels), uint64_t(group)) * split;
    if (rounds > 0x7fffffffull) return DFC_EUNSUPPORTED;
    g.rounds = uint32_t(rounds);
    // one workgroup per round: the hardware hands out the tail
    const uint32_t grid = g.rounds;
    if (split > 1)
        hipLaunchKernelGGL(fill_zero_kernel, dim3(256), dim3(256), 0, stream, g.y, uint64_t(g.batch) * g.rows);
    hipLaunchKernelGGL((dfc_gemm_kernel<C, NT>), dim3(grid), dim3(waves * kWave), lds, stream, g);
    return hipGetLastError() == hipSuccess ? DFC_OK : DFC_EHIP;
}

template <int C>
dfc_status launch_gemm_c(const GemmArgs &g, uint32_t max_block, hipStream_t stream) {
    return g.batch <= 32 ? launch_gemm<C, 1>(g, max_block, stream) : launch_gemm<C, 2>(g, max_block, stream);
}

}  // namespace

extern "C" {

dfc_status dfc_decode_gemm(const void *w_blob_dev, const dfc_info *info, const uint16_t *x_dev, uint32_t batch,
                           float *y_dev, uint32_t *status_dev, void *stream) {
    if (!info || !w_blob_dev || !x_dev || !y_dev) return DFC_EINVAL;
    if (batch < 1 || batch > DFC_GEMM_MAX_BATCH) return DFC_EINVAL;
    if ((reinterpret_cast<uintptr_t>(w_blob_dev) & 255u) || (reinterpret_cast<uintptr_t>(x_dev) & 15u) ||
        (reinterpret_cast<uintptr_t>(y_dev) & 3u))
        return DFC_EINVAL;
    const dfc_info &in = *info;
    if (in.layout != DFC_LAYOUT_PANEL || in.panel_rows != dfc::kPanelRows || in.lanes_per_block != 64)
        return DFC_EUNSUPPORTED;
    const uint32_t C = in.chunk_bytes;
    if (C != 4 && C != 8 && C != 16 && C != 32) return DFC_EINVAL;
    if (in.lut_bits < 8 || in.lut_bits > 12 || in.min_len < 1) return DFC_EINVAL;
    if (in.max_block_elems > 64u * dfc::ceil_div(8ull * C, in.min_len)) return DFC_EINVAL;
    const uint64_t limit = kNowhere - 64u * 1024u;
    if (in.words_bytes > limit || in.offsets_bytes > limit || in.raw_bytes > limit ||
        2ull * DFC_GEMM_MAX_BATCH * in.cols > limit || 4ull * DFC_GEMM_MAX_BATCH * in.rows > limit)
        return DFC_EUNSUPPORTED;
    const uint8_t *base = static_cast<const uint8_t *>(w_blob_dev);
    GemmArgs g;
    std::memset(&g, 0, sizeof(g));
    g.words = reinterpret_cast<const uint32_t *>(base + in.off_words);
    g.offw = reinterpret_cast<const uint32_t *>(base + in.off_offsets);
    g.blockout = reinterpret_cast<const uint32_t *>(base + in.off_blockout);
    g.items = reinterpret_cast<const uint32_t *>(base + in.off_panels);
    g.raw = base + in.off_raw;
    g.tables = base + in.off_tables;
    g.x = x_dev;
    g.y = y_dev;
    g.words_bytes = uint32_t(in.words_bytes);
    g.offw_bytes = uint32_t(in.offsets_bytes);
    g.raw_bytes = uint32_t(in.raw_bytes);
    g.x_bytes = uint32_t(2ull * batch * in.cols);
    g.y_bytes = uint32_t(4ull * batch * in.rows);
    g.n_panels = uint32_t(in.rows / dfc::kPanelRows);
    g.panel_k = in.panel_k;
    g.slices = uint32_t(dfc::ceil_div(in.cols, in.panel_k));
    g.cols = uint32_t(in.cols);
    g.rows = uint32_t(in.rows);
    g.batch = batch;
    g.tables_bytes = uint32_t((in.tables_bytes + 15) & ~15ull);
    g.lut_bits = in.lut_bits;
    g.status = status_dev;
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (C) {
        case 4: return launch_gemm_c<4>(g, in.max_block_elems, st);
        case 8: return launch_gemm_c<8>(g, in.max_block_elems, st);
        case 16: return launch_gemm_c<16>(g, in.max_block_elems, st);
        default: return launch_gemm_c<32>(g, in.max_block_elems, st);
    }
}

}  // extern "C"
