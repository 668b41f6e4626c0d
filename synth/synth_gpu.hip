// GPU copy of the seeded expert-record generator in synth.c.
//
// It writes the same bytes as synth_expert_blob() on the host (same draws,
// same Irwin–Hall normal, same correctly rounded per-row quantiser), so that
// gigabytes of synthetic expert weights can be produced in device memory
// instead of on the host and copied over.  Input preparation only: nothing of
// the layer's own arithmetic is here.
//
// Build: hipcc --offload-arch=gfx950 -O3 -ffp-contract=off -shared -fPIC
#include <hip/hip_runtime.h>
#include <stdint.h>

#define SYN_GOLDEN 0x9E3779B97F4A7C15ULL

__host__ __device__ static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

__device__ static inline uint64_t draw(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * SYN_GOLDEN);
}

__device__ static inline int32_t sum16(uint64_t v) {
  return (int32_t)(v & 0xFFFF) + (int32_t)((v >> 16) & 0xFFFF) +
         (int32_t)((v >> 32) & 0xFFFF) + (int32_t)(v >> 48);
}

__device__ static inline float normal_at(uint64_t key, uint64_t i) {
  int32_t s = sum16(draw(key, 3 * i)) + sum16(draw(key, 3 * i + 1)) +
              sum16(draw(key, 3 * i + 2));
  return (float)(s - 393210) * (1.0f / 65536.0f);
}

static uint64_t host_key(uint64_t seed, uint32_t layer, uint32_t tensor,
                         uint32_t expert, uint32_t matrix) {
  uint64_t k = mix64(seed + SYN_GOLDEN);
  k = mix64(k ^ (((uint64_t)layer << 32) | tensor));
  k = mix64(k ^ (((uint64_t)expert << 32) | matrix));
  return k;
}

struct MatJob {
  uint64_t key[8];   // one key per expert of this launch (<= 8 per launch)
  uint8_t *codes[8]; // first code row of this matrix in each expert record
  float *scales[8];  // first scale of this matrix in each expert record
};

// One block per (row, expert); n floats of the row are drawn into LDS, the
// absmax is reduced, then codes are packed byte by byte.
__global__ void __launch_bounds__(256)
k_synth_rows(MatJob job, int n, int wbits, float sigma) {
  extern __shared__ float wrow[];
  __shared__ float red[256];
  const int row = blockIdx.x, ex = blockIdx.y, tid = threadIdx.x;
  const uint64_t key = job.key[ex];
  float amax = 0.0f;
  for (int c = tid; c < n; c += 256) {
    float w = normal_at(key, (uint64_t)row * (uint64_t)n + (uint64_t)c) * sigma;
    wrow[c] = w;
    amax = fmaxf(amax, fabsf(w));
  }
  red[tid] = amax;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] = fmaxf(red[tid], red[tid + s]);
    __syncthreads();
  }
  amax = red[0];
  const float qdiv = (wbits == 8) ? 127.0f : (wbits == 4) ? 7.0f : 2.0f;
  const int qlo = (wbits == 8) ? -127 : (wbits == 4) ? -8 : -2;
  const int qhi = (wbits == 8) ? 127 : (wbits == 4) ? 7 : 1;
  const float s = amax / qdiv;
  const int per = 8 / wbits;
  const unsigned mask = (1u << wbits) - 1u;
  uint8_t *dst = job.codes[ex] + (size_t)row * (size_t)(n / per);
  for (int j = tid; j < n / per; j += 256) {
    unsigned byte = 0;
    for (int i = 0; i < per; i++) {
      int q = 0;
      if (s != 0.0f) {
        q = (int)roundf(wrow[j * per + i] / s);
        q = q < qlo ? qlo : (q > qhi ? qhi : q);
      }
      byte |= ((unsigned)q & mask) << (wbits * i);
    }
    dst[j] = (uint8_t)byte;
  }
  if (tid == 0) job.scales[ex][row] = s;
}

// MXFP4 records (wbits code -4): the block quantiser of synth.c, one
// thread per block of 32 once the row is in LDS.
__device__ static unsigned fp4_code(float w, int X) {
  const float v = fabsf(ldexpf(w, -X));
  unsigned m;
  if (v <= 0.25f) m = 0;
  else if (v < 0.75f) m = 1;
  else if (v <= 1.25f) m = 2;
  else if (v < 1.75f) m = 3;
  else if (v <= 2.5f) m = 4;
  else if (v < 3.5f) m = 5;
  else if (v <= 5.0f) m = 6;
  else m = 7;
  return m == 0 ? 0u : (m | (w < 0.0f ? 8u : 0u));
}

struct MxJob {
  uint64_t key[8];
  uint8_t *codes[8];   // first code row of this matrix in each record
  uint8_t *scales[8];  // first scale byte of this matrix in each record
};

__global__ void __launch_bounds__(256) k_synth_rows_mx(MxJob job, int n, float sigma) {
  extern __shared__ float wrow[];
  const int row = blockIdx.x, ex = blockIdx.y, tid = threadIdx.x;
  const uint64_t key = job.key[ex];
  for (int c = tid; c < n; c += 256)
    wrow[c] = normal_at(key, (uint64_t)row * (uint64_t)n + (uint64_t)c) * sigma;
  __syncthreads();
  for (int b = tid; b < n / 32; b += 256) {
    const float *w = wrow + 32 * b;
    float amax = 0.0f;
    for (int k = 0; k < 32; k++) amax = fmaxf(amax, fabsf(w[k]));
    int s = 127;
    if (amax > 0.0f) {
      int e;
      frexpf(amax, &e);
      s = e - 1 - 2 + 127;
      s = s < 1 ? 1 : (s > 254 ? 254 : s);
    }
    job.scales[ex][(size_t)row * (n / 32) + b] = (uint8_t)s;
    uint8_t *dst = job.codes[ex] + (size_t)row * (n / 2) + 16 * b;
    for (int j = 0; j < 16; j++)
      dst[j] = (uint8_t)(fp4_code(w[2 * j], s - 127) | (fp4_code(w[2 * j + 1], s - 127) << 4));
  }
}

// FP8 records (wbits code -8): the 128x128 block quantiser of synth.c, one
// workgroup per block: the block's amax from a first pass over its draws,
// then the codes from a second.
__device__ static unsigned fp8_code(float v) {
  const unsigned sign = v < 0.0f ? 0x80u : 0u;
  const float a = fabsf(v);
  unsigned code;
  if (a >= 448.0f) {
    code = 0x7E;
  } else {
    int ex;
    frexpf(a, &ex);
    const int E = ex - 1;
    if (a == 0.0f) {
      code = 0;
    } else if (E < -6) {
      code = (unsigned)rintf(ldexpf(a, 9));
    } else {
      int q = (int)rintf(ldexpf(a, 3 - E));
      int EE = E;
      if (q == 16) {
        q = 8;
        EE++;
      }
      code = ((unsigned)(EE + 7) << 3) | (unsigned)(q - 8);
      if (code > 0x7E) code = 0x7E;
    }
  }
  return code == 0 ? 0u : (sign | code);
}

struct F8Job {
  uint64_t key[8];
  uint8_t *codes[8];  // first code row of this matrix in each record
  float *scales[8];   // first block scale of this matrix in each record
};

__global__ void __launch_bounds__(256) k_synth_blocks_f8(F8Job job, int n, float sigma) {
  __shared__ float red[256];
  const int cb = n / 128, blk = blockIdx.x, ex = blockIdx.y, tid = threadIdx.x;
  const int br = blk / cb, bc = blk % cb;
  const uint64_t key = job.key[ex];
  float amax = 0.0f;
  for (int i = tid; i < 128 * 128; i += 256) {
    const int r = br * 128 + i / 128, c = bc * 128 + i % 128;
    amax = fmaxf(amax, fabsf(normal_at(key, (uint64_t)r * (uint64_t)n + (uint64_t)c) * sigma));
  }
  red[tid] = amax;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (tid < k) red[tid] = fmaxf(red[tid], red[tid + k]);
    __syncthreads();
  }
  const float s = red[0] / 448.0f;
  if (tid == 0) job.scales[ex][blk] = s;
  for (int i = tid; i < 128 * 128; i += 256) {
    const int r = br * 128 + i / 128, c = bc * 128 + i % 128;
    const float w = normal_at(key, (uint64_t)r * (uint64_t)n + (uint64_t)c) * sigma;
    job.codes[ex][(size_t)r * n + c] = (uint8_t)(s != 0.0f ? fp8_code(w / s) : 0u);
  }
}

static int f8_blobs(uint64_t seed, uint32_t layer, const uint32_t *expert_ids, int n_experts,
                    int H, int I, float sigma, void *out, size_t stride, hipStream_t st) {
  if (H % 128 || I % 128) return -1;
  const size_t gate_b = (size_t)I * H;
  const size_t nb = (size_t)(I / 128) * (H / 128);
  const int rows[3] = {I, I, H}, cols[3] = {H, H, I};
  for (int e0 = 0; e0 < n_experts; e0 += 8) {
    const int ne = (n_experts - e0) < 8 ? (n_experts - e0) : 8;
    for (int m = 0; m < 3; m++) {
      F8Job job;
      for (int i = 0; i < 8; i++) {
        const int ei = e0 + (i < ne ? i : 0);
        uint8_t *base = (uint8_t *)out + (size_t)ei * stride;
        float *sc = (float *)(base + 3 * gate_b);
        job.key[i] = host_key(seed, layer, 4u + (uint32_t)m, expert_ids[ei], (uint32_t)m);
        job.codes[i] = base + (size_t)m * gate_b;
        job.scales[i] = sc + (size_t)m * nb;
      }
      hipLaunchKernelGGL(k_synth_blocks_f8, dim3((rows[m] / 128) * (cols[m] / 128), ne),
                         dim3(256), 0, st, job, cols[m], sigma);
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return (int)err;
    }
  }
  return 0;
}

static int mx_blobs(uint64_t seed, uint32_t layer, const uint32_t *expert_ids, int n_experts,
                    int H, int I, float sigma, void *out, size_t stride, hipStream_t st) {
  const size_t gate_b = (size_t)I * H / 2, down_b = (size_t)H * I / 2;
  const int rows[3] = {I, I, H}, cols[3] = {H, H, I};
  for (int e0 = 0; e0 < n_experts; e0 += 8) {
    const int ne = (n_experts - e0) < 8 ? (n_experts - e0) : 8;
    for (int m = 0; m < 3; m++) {
      MxJob job;
      for (int i = 0; i < 8; i++) {
        const int ei = e0 + (i < ne ? i : 0);
        uint8_t *base = (uint8_t *)out + (size_t)ei * stride;
        uint8_t *sb = base + 2 * gate_b + down_b;
        job.key[i] = host_key(seed, layer, 4u + (uint32_t)m, expert_ids[ei], (uint32_t)m);
        job.codes[i] = base + (m == 0 ? 0 : (m == 1 ? gate_b : 2 * gate_b));
        job.scales[i] = sb + (size_t)(m == 0 ? 0 : (m == 1 ? 1 : 2)) * I * (H / 32);
      }
      hipLaunchKernelGGL(k_synth_rows_mx, dim3(rows[m], ne), dim3(256), sizeof(float) * cols[m],
                         st, job, cols[m], sigma);
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return (int)err;
    }
  }
  return 0;
}

extern "C" {

// Fills the records of experts expert_ids[0..n_experts) of (seed, layer) at
// out + i*stride (device memory, caller-owned).  Same bytes as
// synth_expert_blob() on the host.  Returns 0, -1 on bad arguments, or the
// HIP error code.
int synth_gpu_expert_blobs(uint64_t seed, uint32_t layer, const uint32_t *expert_ids,
                           int n_experts, int H, int I, int wbits, float sigma,
                           void *out, size_t stride, void *stream) {
  if ((wbits != 8 && wbits != 4 && wbits != 2 && wbits != -4 && wbits != -8) || H <= 0 ||
      I <= 0 || H % 32 ||
      I % 32 || n_experts < 0 || !out || H > 16384 || I > 16384)
    return -1;
  hipStream_t st = (hipStream_t)stream;
  if (wbits == -4) return mx_blobs(seed, layer, expert_ids, n_experts, H, I, sigma, out, stride, st);
  if (wbits == -8) return f8_blobs(seed, layer, expert_ids, n_experts, H, I, sigma, out, stride, st);
  const size_t gate_b = (size_t)I * H * wbits / 8;
  const size_t down_b = (size_t)H * I * wbits / 8;
  const int rows[3] = {I, I, H}, cols[3] = {H, H, I};
  for (int e0 = 0; e0 < n_experts; e0 += 8) {
    const int ne = (n_experts - e0) < 8 ? (n_experts - e0) : 8;
    for (int m = 0; m < 3; m++) {
      MatJob job;
      for (int i = 0; i < 8; i++) {
        const int ei = e0 + (i < ne ? i : 0);
        uint8_t *base = (uint8_t *)out + (size_t)ei * stride;
        float *scales = (float *)(base + 2 * gate_b + down_b);
        job.key[i] = host_key(seed, layer, 4u + (uint32_t)m, expert_ids[ei], (uint32_t)m);
        job.codes[i] = base + (m == 0 ? 0 : (m == 1 ? gate_b : 2 * gate_b));
        job.scales[i] = scales + (m == 0 ? 0 : (m == 1 ? I : 2 * I));
      }
      dim3 grid(rows[m], ne);
      hipLaunchKernelGGL(k_synth_rows, grid, dim3(256), sizeof(float) * cols[m], st,
                         job, cols[m], wbits, sigma);
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return (int)err;
    }
  }
  return 0;
}

}  // extern "C"
