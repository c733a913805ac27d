// Upload of the small per-launch cloud tables of ragged batches.
#include <algorithm>

#include "segments.h"

namespace pointops {

constexpr int kUploadWords = 240;  // 1920 bytes of kernel arguments per launch

struct UploadChunk {
    int64_t v[kUploadWords];
};

__global__ __launch_bounds__(256) void upload_words_kernel(UploadChunk c, int n,
                                                           int64_t* __restrict__ dst) {
    if ((int)threadIdx.x < n) dst[threadIdx.x] = c.v[threadIdx.x];
}

hipError_t upload_words(const int64_t* host, int64_t n, int64_t* dev, hipStream_t stream) {
    for (int64_t i = 0; i < n; i += kUploadWords) {
        const int m = (int)std::min<int64_t>(kUploadWords, n - i);
        UploadChunk c{};
        std::copy(host + i, host + i + m, c.v);
        hipLaunchKernelGGL(upload_words_kernel, dim3(1), dim3(256), 0, stream, c, m, dev + i);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace pointops
