/*
 * Seeded synthetic KV payload: byte content of every row of every layer.
 *
 * Word w (8 bytes, little endian) of row (layer, req, pos) is
 *     mix64(seed XOR pack(layer, req, pos, w))
 * where mix64 is the SplitMix64 output function (Steele, Lea & Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014, with the
 * 64-bit finaliser constants published with Vigna's splitmix64) and pack puts
 * layer in bits 63..56, req in 55..40, pos in 39..16 and w in 15..0.
 *
 * This is input generation only.  It holds none of the resolver's arithmetic,
 * and both the GPU path and the CPU reference read what it writes.
 */
#include <pthread.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t mix64(uint64_t x)
{
    uint64_t z = x + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static inline uint64_t pack(uint64_t layer, uint64_t req, uint64_t pos, uint64_t w)
{
    return (layer << 56) | (req << 40) | (pos << 16) | w;
}

/* One contiguous run of rows: n_rows positions pos0, pos0+1, ... of (layer, req),
 * written at dst, dst + stride, ... */
typedef struct synth_seg {
    uint8_t *dst;
    int64_t n_rows;
    int64_t stride;
    int64_t layer;
    int64_t req;
    int64_t pos0;
} synth_seg;

static void fill_seg(const synth_seg *s, int32_t row_bytes, uint64_t seed)
{
    const int32_t words = row_bytes / 8;
    for (int64_t i = 0; i < s->n_rows; ++i) {
        uint8_t *row = s->dst + i * s->stride;
        const uint64_t pos = (uint64_t)(s->pos0 + i);
        for (int32_t w = 0; w < words; ++w) {
            uint64_t v = mix64(seed ^ pack((uint64_t)s->layer, (uint64_t)s->req, pos, (uint64_t)w));
            memcpy(row + 8 * (int64_t)w, &v, 8);
        }
    }
}

typedef struct job {
    const synth_seg *segs;
    int64_t n_segs;
    int32_t row_bytes;
    uint64_t seed;
    int tid, nthreads;
} job;

static void *run_job(void *arg)
{
    const job *j = (const job *)arg;
    for (int64_t i = j->tid; i < j->n_segs; i += j->nthreads)
        fill_seg(&j->segs[i], j->row_bytes, j->seed);
    return NULL;
}

/* Fill every segment; returns 0, or -1 on bad arguments. */
int synth_fill_segments(const synth_seg *segs, int64_t n_segs, int32_t row_bytes,
                        uint64_t seed, int32_t nthreads)
{
    if (row_bytes <= 0 || row_bytes % 8 != 0 || n_segs < 0)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 64)
        nthreads = 64;
    if (n_segs < nthreads)
        nthreads = n_segs > 0 ? (int32_t)n_segs : 1;
    pthread_t th[64];
    job jobs[64];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (job){segs, n_segs, row_bytes, seed, t, nthreads};
    }
    for (int t = 1; t < nthreads; ++t)
        pthread_create(&th[t], NULL, run_job, &jobs[t]);
    run_job(&jobs[0]);
    for (int t = 1; t < nthreads; ++t)
        pthread_join(th[t], NULL);
    return 0;
}
