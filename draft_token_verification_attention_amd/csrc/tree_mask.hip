// tree_mask.hip -- token tree -> ancestor-or-self bit rows, depths, position ids.
//
// "Speculative decoding" (Zero to Frontier textbook, ch. 20, section 20.5), box
// "Token tree and tree attention" and the exercise "The tree attention mask": node i
// sees every prefix position, itself and its ancestors; depth = number of ancestors;
// position id = prefix length + depth.
//
// One wave per row: all lanes walk the (short) ancestor chain together, reading the
// same parent entries, and each lane owns a run of the row's words, so every row is
// written with coalesced stores.  Block 0 also validates the whole parent array and
// writes the status word (0, or 1 + the first node whose parent is not in [-1, i)).
// A walk that meets an invalid parent stops there, so every wave terminates.
#include "sv_common.h"

namespace {

constexpr int kMaskThreads = 256;
constexpr int kMaskWaves = kMaskThreads / sv::kWave;

__global__ __launch_bounds__(kMaskThreads) void tree_mask_kernel(const int32_t *__restrict__ parents, int32_t n,
                                                                 int32_t prefix_len, int32_t words,
                                                                 uint32_t *__restrict__ bits,
                                                                 int32_t *__restrict__ depth,
                                                                 int64_t *__restrict__ pos,
                                                                 int32_t *__restrict__ status)
{
    __shared__ int first_bad;
    const int lane = threadIdx.x % sv::kWave;
    const int wave = threadIdx.x / sv::kWave;

    if (blockIdx.x == 0) {
        if (threadIdx.x == 0) first_bad = n;
        __syncthreads();
        for (int i = threadIdx.x; i < n; i += kMaskThreads) {
            const int p = parents[i];
            if (p < -1 || p >= i) atomicMin(&first_bad, i);
        }
        __syncthreads();
        if (threadIdx.x == 0) *status = first_bad < n ? first_bad + 1 : 0;
    }

    const int row_stride = gridDim.x * kMaskWaves;
    for (int i = blockIdx.x * kMaskWaves + wave; i < n; i += row_stride) {
        uint32_t *row = bits + (int64_t)i * words;
        for (int w = lane; w < words; w += sv::kWave) row[w] = 0u;
        // The ancestor chain strictly decreases while parents are valid, so this loop
        // ends after at most i + 1 steps; an invalid parent ends it early.
        int d = 0;
        int j = i;
        while (true) {
            const int w = j >> 5;
            if ((w & (sv::kWave - 1)) == lane) {
                // each lane owns words lane, lane+64, ...: plain read-modify-write
                row[w] |= 1u << (j & 31);
            }
            const int p = parents[j];
            if (p < 0 || p >= j) break;
            j = p;
            ++d;
        }
        if (lane == 0) {
            depth[i] = d;
            pos[i] = (int64_t)prefix_len + d;
        }
    }
}

}  // namespace

extern "C" sv_status sv_build_tree_mask(const int32_t *parents, int32_t n, int32_t prefix_len, uint32_t *bits,
                                        int32_t *depth, int64_t *pos, int32_t *dev_status, void *stream)
{
    if (!parents || !bits || !depth || !pos || !dev_status) return SV_ERR_INVALID_ARG;
    if (n < 1 || prefix_len < 0) return SV_ERR_INVALID_ARG;
    const int32_t words = (n + 31) / 32;
    int blocks = (n + kMaskWaves - 1) / kMaskWaves;
    if (blocks > 2048) blocks = 2048;
    (void)hipGetLastError();
    hipLaunchKernelGGL(tree_mask_kernel, dim3(blocks), dim3(kMaskThreads), 0, (hipStream_t)stream, parents, n,
                       prefix_len, words, bits, depth, pos, dev_status);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

extern "C" const char *sv_status_string(sv_status status)
{
    switch (status) {
    case SV_OK: return "SV_OK";
    case SV_ERR_INVALID_ARG: return "SV_ERR_INVALID_ARG";
    case SV_ERR_UNSUPPORTED: return "SV_ERR_UNSUPPORTED";
    case SV_ERR_WORKSPACE: return "SV_ERR_WORKSPACE";
    case SV_ERR_HIP: return "SV_ERR_HIP";
    }
    return "SV_UNKNOWN_STATUS";
}
