/* Seeded synthetic inputs: a counter-based generator (splitmix64) that fills
 * bf16 weight tensors and token-id arrays.  Same definition as synth/gen.py,
 * which is the slow numpy version; both must give identical bits.
 *
 *   base(seed, tid) = mix64(seed * 2^32 + tid)
 *   h_i             = mix64(base + (i + 1) * 0x9E3779B97F4A7C15)     (mod 2^64)
 *   c_i             = (h_i & 0xFFFF) + (h_i>>16 & 0xFFFF) + (h_i>>32 & 0xFFFF) + (h_i>>48) - 131070
 *   weight_i        = bf16_rne( fl32( fl32(c_i) * k ) + mean )  with k = fl32(std / sqrt((2^32-1)/3))
 *   token_i         = ((h_i >> 32) * vocab) >> 32
 *
 * mix64 is the splitmix64 output function (Steele, Lea, Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014; constants as in
 * Vigna's public-domain splitmix64.c).  c_i is an Irwin-Hall sum of four
 * 16-bit uniforms, centred: mean 0, variance (2^32-1)/3.
 */
#include <stdint.h>
#include <string.h>
#include <pthread.h>

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t r = 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)((u + r) >> 16);
}

typedef struct {
  uint64_t base, i0, i1;
  float k, mean;
  uint16_t* out;
  int32_t* tok;
  int64_t vocab;
} job_t;

static void* fill_bf16_job(void* p) {
  job_t* j = (job_t*)p;
  for (uint64_t i = j->i0; i < j->i1; ++i) {
    uint64_t h = mix64(j->base + (i + 1) * 0x9E3779B97F4A7C15ull);
    int32_t c = (int32_t)((h & 0xFFFF) + ((h >> 16) & 0xFFFF) + ((h >> 32) & 0xFFFF) + (h >> 48)) - 131070;
    float w = (float)c * j->k; /* one IEEE fp32 multiply (built with -ffp-contract=off) */
    float v = w + j->mean;     /* one IEEE fp32 add (exact when mean == 0) */
    j->out[i - j->i0] = f32_to_bf16_rne(v);
  }
  return 0;
}

static void* fill_tok_job(void* p) {
  job_t* j = (job_t*)p;
  for (uint64_t i = j->i0; i < j->i1; ++i) {
    uint64_t h = mix64(j->base + (i + 1) * 0x9E3779B97F4A7C15ull);
    j->tok[i - j->i0] = (int32_t)(((h >> 32) * (uint64_t)j->vocab) >> 32);
  }
  return 0;
}

static void run(job_t* proto, uint64_t start, uint64_t n, int nthreads, int is_tok) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  if (n < (uint64_t)nthreads * 65536) nthreads = 1;
  pthread_t th[64];
  job_t jobs[64];
  uint64_t per = (n + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = *proto;
    uint64_t a = start + (uint64_t)t * per, b = a + per;
    if (a > start + n) a = start + n;
    if (b > start + n) b = start + n;
    jobs[t].i0 = a;
    jobs[t].i1 = b;
    if (is_tok) jobs[t].tok = proto->tok + (a - start);
    else jobs[t].out = proto->out + (a - start);
    if (nthreads == 1) { is_tok ? fill_tok_job(&jobs[t]) : fill_bf16_job(&jobs[t]); }
    else pthread_create(&th[t], 0, is_tok ? fill_tok_job : fill_bf16_job, &jobs[t]);
  }
  if (nthreads > 1)
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], 0);
}

uint64_t synth_stream_base(uint64_t seed, uint64_t tid) { return mix64((seed << 32) + tid); }

/* Elements [start, start+n) of tensor (seed, tid) into out[0..n). */
void synth_fill_bf16(uint64_t seed, uint64_t tid, uint64_t start, uint64_t n, float k, float mean,
                     uint16_t* out, int nthreads) {
  job_t j;
  memset(&j, 0, sizeof j);
  j.base = synth_stream_base(seed, tid);
  j.k = k;
  j.mean = mean;
  j.out = out;
  run(&j, start, n, nthreads, 0);
}

void synth_fill_tokens(uint64_t seed, uint64_t tid, uint64_t start, uint64_t n, int64_t vocab,
                       int32_t* out, int nthreads) {
  job_t j;
  memset(&j, 0, sizeof j);
  j.base = synth_stream_base(seed, tid);
  j.vocab = vocab;
  j.tok = out;
  run(&j, start, n, nthreads, 1);
}
