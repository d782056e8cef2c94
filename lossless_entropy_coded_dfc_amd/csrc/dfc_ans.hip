// dfc_ans.hip - gfx950 decoder for containers in the interleaved rANS layout
// (DFC_LAYOUT_ANS; the code and the container are stated in dfc.h).
//
// The exponents are coded with rANS, an arithmetic-family code (DFloat11
// blog, section 02; the VcLLM page's introduction describes an ANS decoder);
// sign and mantissa are one raw byte per value as in the Huffman layouts.
//
// One wavefront decodes one block: lane l holds the state of the block's
// lane l and decodes elements i * 64 + l, one step i at a time.  Per step:
// the slot table (derived from the frequencies into LDS by every workgroup,
// 16 KB) gives symbol, frequency and
// cumulative count; the lanes whose state drops below 2^16 take the block's
// next 16-bit words in lane order (ballot, then each lane's rank among them),
// read from a per-wavefront ring of 1024 words in LDS.  A round of eight
// steps consumes at most 512 words, so the ring is refilled only between
// rounds, 512 words at a time from registers loaded one refill ahead: the
// loop waits for a word load only there, and the eight steps of a round run
// with no memory waits.  Word and raw-byte loads stop at the block's end, so
// no block fetches another's bytes.  Only a block's last step tests which lanes take
// part.  The
// step's 64 exponent bytes go to an LDS stage; every 8 steps the stage holds
// 512 consecutive exponents, which the lanes merge with the raw bytes (loaded
// one round ahead) into bf16 octets and write with 16-byte stores (1 KB
// contiguous per instruction).  At the end every lane's state must be back
// at 2^16 and the block's words consumed exactly, else the status word is
// set.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <type_traits>
#include <vector>

#include "dfc.h"
#include "dfc_ans_launch.h"
#include "dfc_decode_core.h"
#include "dfc_format.h"

namespace {

constexpr uint32_t kAnsWaves = 8;  // wavefronts per workgroup, one block each
constexpr uint32_t kRing = 1024;   // words of a wavefront's LDS ring
constexpr uint32_t kSeg = 512;     // words per ring refill (eight per lane)

struct AnsItem {
    const uint16_t *words;     // all blocks' word streams
    const uint32_t *offsets;   // first word of every block, n_blocks + 1
    const uint32_t *states;    // 64 initial states per block
    const uint8_t *raw;        // raw bytes, padded to 16
    const uint16_t *freqs;     // quantised frequencies f[256] (sum 4096)
    const uint32_t *table;     // slot table from dfc_derive_tables, or null: derive it here
    uint16_t *dst;
    uint32_t words_bytes, states_bytes, raw_bytes, dst_bytes;
    uint32_t n, n_blocks, steps;
    uint32_t wg_begin;  // first workgroup of this item in the grid
};

struct AnsBatch {
    AnsItem item[DFC_MAX_BATCH];
    uint32_t count;
    uint32_t *status;
};

__global__ __launch_bounds__(kAnsWaves * kWave) void dfc_ans_kernel(const AnsBatch args) {
    __shared__ __align__(16) uint32_t table[dfc::kAnsSlots];
    __shared__ __align__(16) uint8_t stage_all[kAnsWaves][512];
    // the ring's first 64 words are mirrored after its end, so a word index
    // (start mod kRing) + rank needs no wrap
    __shared__ __align__(16) uint16_t ring_all[kAnsWaves][kRing + kWave];
    const uint32_t wg = blockIdx.x;
    uint32_t it = 0;
    for (uint32_t k = 1; k < args.count; ++k)
        if (wg >= args.item[k].wg_begin) it = k;
    const AnsItem a = args.item[it];

    // the slot table: prepared, or derived from the frequencies (the stage
    // areas serve as scratch)
    if (a.table) {
        for (uint32_t o = threadIdx.x; o < dfc::kAnsSlots / 4; o += blockDim.x)
            reinterpret_cast<uint4 *>(table)[o] = reinterpret_cast<const uint4 *>(a.table)[o];
        __syncthreads();
    } else {
        derive_slot_table(table, &stage_all[0][0], a.freqs);
    }

    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t lane = threadIdx.x % kWave;
    const uint32_t b = (wg - a.wg_begin) * kAnsWaves + wave;
    if (b >= a.n_blocks) return;
    uint8_t *stage = stage_all[wave];
    uint16_t *ring = ring_all[wave];

    const __amdgpu_buffer_rsrc_t words =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(a.words), 0, int(a.words_bytes), kBufferConfig);
    const __amdgpu_buffer_rsrc_t states =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t *>(a.states), 0, int(a.states_bytes), kBufferConfig);
    const __amdgpu_buffer_rsrc_t raw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(a.raw), 0, int(a.raw_bytes), kBufferConfig);
    const __amdgpu_buffer_rsrc_t dst = __builtin_amdgcn_make_buffer_rsrc(a.dst, 0, int(a.dst_bytes), kBufferConfig);
    const const_u32_ptr offsets = (const_u32_ptr)(a.offsets);

    const uint32_t per = kWave * a.steps;
    const uint32_t e0 = b * per;                 // first element of the block (a multiple of 8)
    const uint32_t cnt = min(per, a.n - e0);     // elements in the block
    const uint32_t nsteps = (cnt + kWave - 1) / kWave;
    const uint32_t w_begin = offsets[b], w_end = offsets[b + 1];

    uint32_t x = __builtin_amdgcn_raw_buffer_load_b32(states, 4u * (b * kWave + lane), 0, 0);
    // ring: words [base, base + kRing) at ring[word mod kRing], base a
    // multiple of 8; pend: words [base + kRing, base + kRing + kSeg), eight
    // per lane
    uint32_t base = w_begin & ~7u, off = w_begin & 7u;
    // eight words from word w on; none (zeros, no memory access) from the
    // block's end on, so the ring never reads the next block's words
    auto load8 = [&](uint32_t w) {
        return __builtin_amdgcn_raw_buffer_load_b128(words, w < w_end ? 2u * w : kNowhere, 0, 0);
    };
    // raw bytes of the octet at block-relative element q; none past the block
    auto load_raw = [&](uint32_t q) {
        return __builtin_amdgcn_raw_buffer_load_b64(raw, q < cnt ? e0 + q : kNowhere, 0, 0);
    };
    // eight words at ring slot p (a multiple of 8), and their mirror
    auto put8 = [&](uint32_t p, const u32x4 &v) {
        *reinterpret_cast<u32x4 *>(ring + p) = v;
        if (p < kWave) *reinterpret_cast<u32x4 *>(ring + kRing + p) = v;
    };
#pragma unroll
    for (uint32_t q = 0; q < kRing; q += kSeg)
        put8((base + q + 8u * lane) & (kRing - 1u), load8(base + q + 8u * lane));
    u32x4 pend = load8(base + kRing + 8u * lane);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // raw bytes of the first round's octet (512 elements per round)
    u32x2 R = load_raw(8u * lane);

    // One step: every lane decodes its element of step i.  Only the block's
    // last step can be partial, so only it tests which lanes take part.
    auto step = [&](uint32_t i, auto tail) {
        constexpr bool kTail = decltype(tail)::value;
        const bool live = !kTail || i * kWave + lane < cnt;
        const uint32_t e = table[x & (dfc::kAnsSlots - 1u)];
        const uint32_t f = ((e >> 8) & 0xFFFu) + 1u;
        const uint32_t xn = f * (x >> dfc::kAnsProbBits) + (e >> 20);  // e >> 20 = slot - cum
        const bool need = live && xn < uint32_t(dfc::kAnsLow);
        const uint64_t m = __builtin_amdgcn_ballot_w64(need);
        // this lane's word: the next unread word's slot + the lane's rank
        const uint32_t rank = __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
        const uint16_t *next = ring + ((base + off) & (kRing - 1u));
        const uint32_t w = next[rank];
        if constexpr (kTail)
            x = need ? (xn << 16) | w : (live ? xn : x);
        else
            x = need ? (xn << 16) | w : xn;
        stage[(i & 7u) * kWave + lane] = uint8_t(e);
        off += uint32_t(__builtin_popcountll(m));
    };
    // Round r (steps 8r .. 8r + 7) is staged: merge with its raw bytes, store.
    auto flush = [&](uint32_t r) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const u32x2 E = *reinterpret_cast<const u32x2 *>(stage + 8u * lane);
        const u32x4 o = assemble8(E, R);
        const uint32_t first = 512u * r + 8u * lane;  // block-relative element of this octet
        const uint32_t h = e0 / 8u + 64u * r + lane;   // octet index in the output
        __builtin_amdgcn_raw_buffer_store_b128(o, dst, first + 8u <= cnt ? 16u * h : kNowhere, 0, 0);
        if (cnt - 512u * r < 512u && (cnt & 7u)) {
            // the block's last round ends inside an octet: its values one by one
            const uint32_t v[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const bool in = first + 8u > cnt && first + uint32_t(j) < cnt;
                __builtin_amdgcn_raw_buffer_store_b16(uint16_t(v[j >> 1] >> (16 * (j & 1))), dst,
                                                      in ? 2u * (8u * h + uint32_t(j)) : kNowhere, 0, 0);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        R = load_raw(512u * (r + 1u) + 8u * lane);
    };

    // Whole rounds: eight steps consume at most 512 words, so the ring (which
    // holds at least kRing - kSeg words ahead at a round's start) needs
    // refilling only between rounds, and then by one segment.
    // The flush comes first: its wait for R (loaded by the previous flush)
    // then never has to cover this round's refill load, and the refill's
    // wait for pend (loaded a refill earlier) lets the flush's stores run.
    const uint32_t rounds = (cnt / kWave) / 8u;
    wait_for(x);
    for (uint32_t r = 0; r < rounds; ++r) {
        // decode steps at a raised wave priority, the flush at the normal one
        // (wavefronts that are decoding issue first; 1-2% in one-process timing)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (uint32_t j = 0; j < 8u; ++j) step(8u * r + j, std::false_type{});
        __builtin_amdgcn_s_setprio(0);
        flush(r);
        if (off >= kSeg) {
            // words [base, base + kSeg) are consumed: their slots take pend
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            put8((base + kRing + 8u * lane) & (kRing - 1u), pend);
            base += kSeg;
            off -= kSeg;
            pend = load8(base + kRing + 8u * lane);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }
    // The last, partial round.
    if (8u * rounds < nsteps) {
        for (uint32_t i = 8u * rounds; i < nsteps; ++i) {
            if (i < cnt / kWave)
                step(i, std::false_type{});
            else
                step(i, std::true_type{});
        }
        flush(rounds);
    }
    // every lane back at the encoder's starting state, every word consumed
    const bool bad = (base + off != w_end) | (__builtin_amdgcn_ballot_w64(x != uint32_t(dfc::kAnsLow)) != 0);
    if (bad && lane == 0 && args.status) atomicOr(args.status, kStatusCorrupt);
}

// The slot table as the decoder derives it, copied out (for inspection).
__global__ __launch_bounds__(1024) void derive_slot_table_kernel(const uint16_t *freqs, uint32_t *dst) {
    __shared__ __align__(16) uint32_t table[dfc::kAnsSlots];
    __shared__ __align__(16) uint8_t scratch[kSlotScratchBytes];
    derive_slot_table(table, scratch, freqs);
    for (uint32_t o = threadIdx.x; o < dfc::kAnsSlots / 4; o += blockDim.x)
        reinterpret_cast<uint4 *>(dst)[o] = reinterpret_cast<const uint4 *>(table)[o];
}

}  // namespace

namespace dfc {

dfc_status ans_derive_tables(const void *blob_dev, const dfc_info &info, uint32_t threads, void *dst,
                             hipStream_t stream) {
    const uint16_t *freqs = reinterpret_cast<const uint16_t *>(static_cast<const uint8_t *>(blob_dev) + info.off_tables);
    derive_slot_table_kernel<<<dim3(1), dim3(threads), 0, stream>>>(freqs, static_cast<uint32_t *>(dst));
    return hipGetLastError() == hipSuccess ? DFC_OK : DFC_EHIP;
}

dfc_status ans_check_item(const dfc_batch_item &it) {
    const dfc_info &in = *it.info;
    if (in.lanes_per_block != kAnsLanes || in.ans_prob_bits != kAnsProbBits) return DFC_EUNSUPPORTED;
    if (in.ans_steps < 8 || in.ans_steps > 65536 || in.ans_steps % 8) return DFC_EINVAL;
    const uint64_t limit = kNowhere - 64u * 1024u;
    if (2 * in.n > limit || in.words_bytes > limit || in.blockout_bytes > limit || in.raw_bytes > limit)
        return DFC_EUNSUPPORTED;
    return DFC_OK;
}

dfc_status ans_launch(const dfc_batch_item *items, const uint32_t *idx, uint32_t count, uint32_t *status,
                      hipStream_t stream) {
    AnsBatch args;
    std::memset(&args, 0, sizeof(args));
    uint32_t wg = 0, m = 0;
    for (uint32_t k = 0; k < count; ++k) {
        const dfc_batch_item &bi = items[idx[k]];
        const dfc_info &in = *bi.info;
        if (in.n_blocks == 0) continue;
        const uint8_t *base = static_cast<const uint8_t *>(bi.blob_dev);
        AnsItem &a = args.item[m++];
        a.words = reinterpret_cast<const uint16_t *>(base + in.off_words);
        a.offsets = reinterpret_cast<const uint32_t *>(base + in.off_offsets);
        a.states = reinterpret_cast<const uint32_t *>(base + in.off_blockout);
        a.raw = base + in.off_raw;
        a.freqs = reinterpret_cast<const uint16_t *>(base + in.off_tables);
        a.table = static_cast<const uint32_t *>(bi.tables_dev);
        a.dst = bi.dst_dev;
        a.words_bytes = uint32_t(in.words_bytes);
        a.states_bytes = uint32_t(in.blockout_bytes);
        a.raw_bytes = uint32_t(in.raw_bytes);
        a.dst_bytes = uint32_t(2 * in.n);
        a.n = uint32_t(in.n);
        a.n_blocks = uint32_t(in.n_blocks);
        a.steps = in.ans_steps;
        a.wg_begin = wg;
        wg += uint32_t(ceil_div(in.n_blocks, kAnsWaves));
    }
    if (!m) return DFC_OK;
    args.count = m;
    args.status = status;
    dfc_ans_kernel<<<dim3(wg), dim3(kAnsWaves * kWave), 0, stream>>>(args);
    return hipGetLastError() == hipSuccess ? DFC_OK : DFC_EHIP;
}

}  // namespace dfc
