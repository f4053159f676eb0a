// gs_sort_keys: stable least-significant-digit radix sort of 64-bit keys with
// 32-bit payloads, 8-bit digits (the GPU radix sort of reference [22] of "A
// Scalable PyTorch Abstraction for Multi-GPU Gaussian Splatting").
//
// Each pass over one digit runs three steps:
//   1. k_radix_hist    per-block digit histogram (LDS counters), written
//                      digit-major: hist[digit * n_blocks + block]
//   2. prefix sum      of that array: the first output slot of every
//                      (digit, block)
//   3. k_radix_scatter each wave ranks its keys stably: lanes holding the same
//                      digit are found with 8 ballots (one per digit bit), the
//                      rank is the count of such lanes below, plus a per-wave
//                      running count per digit in LDS; waves then offset each
//                      other per digit and every key goes to its slot.
// A block holds 2048 keys: 4 waves x 8 rounds x 64 lanes, each wave a
// contiguous 512-key run, so block order = wave order = round order = lane
// order and the sort is stable.
#include "internal.h"

namespace gs {

constexpr int SORT_THREADS = 256;
constexpr int SORT_ROUNDS = 8;
constexpr int SORT_WAVE_KEYS = 64 * SORT_ROUNDS;
constexpr int SORT_TILE = SORT_THREADS * SORT_ROUNDS;

__global__ __launch_bounds__(SORT_THREADS) void k_radix_hist(const uint64_t* __restrict__ keys, uint64_t n_keys,
                                                             int shift, uint32_t n_blocks,
                                                             uint32_t* __restrict__ hist)
{
    __shared__ uint32_t cnt[256];
    cnt[threadIdx.x] = 0u;
    __syncthreads();
    const uint64_t base = (uint64_t)blockIdx.x * SORT_TILE;
#pragma unroll
    for (int r = 0; r < SORT_ROUNDS; ++r) {
        const uint64_t i = base + (uint64_t)r * SORT_THREADS + threadIdx.x;
        if (i < n_keys) atomicAdd(&cnt[(uint32_t)(keys[i] >> shift) & 255u], 1u);
    }
    __syncthreads();
    hist[(uint64_t)threadIdx.x * n_blocks + blockIdx.x] = cnt[threadIdx.x];
}

__global__ __launch_bounds__(SORT_THREADS) void k_radix_scatter(const uint64_t* __restrict__ keys_in,
                                                                const uint32_t* __restrict__ vals_in,
                                                                uint64_t* __restrict__ keys_out,
                                                                uint32_t* __restrict__ vals_out, uint64_t n_keys,
                                                                int shift, uint32_t n_blocks,
                                                                const uint32_t* __restrict__ first_slot)
{
    __shared__ uint32_t wcnt[4][256];
    __shared__ uint32_t wbase[4][256];
    const uint32_t wave = threadIdx.x >> 6;
#pragma unroll
    for (int w = 0; w < 4; ++w) wcnt[w][threadIdx.x] = 0u;
    __syncthreads();

    const uint64_t wstart = (uint64_t)blockIdx.x * SORT_TILE + (uint64_t)wave * SORT_WAVE_KEYS;
    uint64_t k[SORT_ROUNDS];
    uint32_t val[SORT_ROUNDS], rank[SORT_ROUNDS], dig[SORT_ROUNDS];
#pragma unroll
    for (int r = 0; r < SORT_ROUNDS; ++r) {
        const uint64_t i = wstart + (uint64_t)r * 64 + lane_id();
        const bool valid = i < n_keys;
        k[r] = valid ? keys_in[i] : 0ull;
        val[r] = valid ? vals_in[i] : 0u;
        const uint32_t d = (uint32_t)(k[r] >> shift) & 255u;
        dig[r] = d;
        uint64_t peers = ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const bool bit = (d >> b) & 1u;
            const uint64_t m = ballot(bit);
            peers &= bit ? m : ~m;
        }
        const uint32_t below = mask_rank(peers);
        const uint32_t prior = wcnt[wave][d];
        rank[r] = prior + below;
        // all lanes have read the counter (LDS is in order within a wave)
        asm volatile("" ::: "memory");
        if (valid && below == 0u) wcnt[wave][d] = prior + (uint32_t)__popcll(peers);
        asm volatile("" ::: "memory");
    }
    __syncthreads();
    {
        const uint32_t d = threadIdx.x;
        uint32_t run = first_slot[(uint64_t)d * n_blocks + blockIdx.x];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            wbase[w][d] = run;
            run += wcnt[w][d];
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < SORT_ROUNDS; ++r) {
        const uint64_t i = wstart + (uint64_t)r * 64 + lane_id();
        if (i < n_keys) {
            const uint32_t pos = wbase[wave][dig[r]] + rank[r];
            if (pos >= n_keys) continue;  // unreachable when the counts are consistent
            keys_out[pos] = k[r];
            vals_out[pos] = val[r];
        }
    }
}

static uint32_t sort_blocks(uint64_t n_keys) { return (uint32_t)((n_keys + SORT_TILE - 1) / SORT_TILE); }

}  // namespace gs

using namespace gs;

extern "C" {

// The histogram holds 256 * n_blocks counters plus the total the prefix sum
// appends after them.
static size_t hist_bytes(uint64_t hist_n) { return (size_t)(((hist_n + 1) * sizeof(uint32_t) + 255) / 256 * 256); }

size_t gs_sort_workspace_bytes(uint64_t n_keys)
{
    const uint64_t hist = 256ull * sort_blocks(n_keys);
    return hist_bytes(hist) + scan_workspace_bytes(hist);
}

gs_status gs_sort_keys(uint64_t* keys, uint32_t* vals, uint64_t* keys_alt, uint32_t* vals_alt, uint64_t n_keys,
                       int32_t end_bit, void* ws, size_t ws_bytes, int32_t* result_in_alt, void* stream)
{
    if (!result_in_alt || end_bit < 1 || end_bit > 64) return GS_ERR_INVALID_ARGUMENT;
    if (n_keys >= ((uint64_t)1 << 32)) return GS_ERR_INVALID_ARGUMENT;
    *result_in_alt = 0;
    if (n_keys == 0) return GS_OK;
    if (!keys || !vals || !keys_alt || !vals_alt || !ws) return GS_ERR_INVALID_ARGUMENT;
    if (ws_bytes < gs_sort_workspace_bytes(n_keys)) return GS_ERR_INVALID_ARGUMENT;
    hipStream_t s = (hipStream_t)stream;
    const uint32_t nb = sort_blocks(n_keys);
    const uint64_t hist_n = 256ull * nb;
    uint32_t* hist = (uint32_t*)ws;
    void* scan_ws = (char*)ws + hist_bytes(hist_n);
    uint64_t *kin = keys, *kout = keys_alt;
    uint32_t *vin = vals, *vout = vals_alt;
    int passes = 0;
    for (int shift = 0; shift < end_bit; shift += 8, ++passes) {
        hipLaunchKernelGGL(k_radix_hist, dim3(nb), dim3(SORT_THREADS), 0, s, kin, n_keys, shift, nb, hist);
        if (hipGetLastError() != hipSuccess) return GS_ERR_HIP;
        if (scan_u32(hist, hist, hist_n, nullptr, scan_ws, s) != hipSuccess) return GS_ERR_HIP;
        hipLaunchKernelGGL(k_radix_scatter, dim3(nb), dim3(SORT_THREADS), 0, s, kin, vin, kout, vout, n_keys, shift,
                           nb, hist);
        if (hipGetLastError() != hipSuccess) return GS_ERR_HIP;
        uint64_t* tk = kin; kin = kout; kout = tk;
        uint32_t* tv = vin; vin = vout; vout = tv;
    }
    *result_in_alt = passes & 1;
    return GS_OK;
}

}  // extern "C"
