/*
 * Reference ("oracle") implementation of the gated delta rule prefill scan:
 * a plain, slow, token-by-token CPU recurrence, in fp64 and in fp32.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or constant with the HIP library; it is built with
 * -O2 -ffp-contract=off and no fast-math so its results are reproducible.
 *
 * Defining ORACLE_MUTANT=n at build time plants one known mistake (used only
 * by the test that checks the pins can tell a wrong oracle from a right one).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

#define REAL double
#define SFX(name) name##_f64
#define RSQRT_EPS(x) (1.0 / sqrt((x) + 1e-6))
#include "gdn_oracle_body.h"
#undef REAL
#undef SFX
#undef RSQRT_EPS

#define REAL float
#define SFX(name) name##_f32
#define RSQRT_EPS(x) (1.0f / sqrtf((x) + 1e-6f))
#include "gdn_oracle_body.h"
#undef REAL
#undef SFX
#undef RSQRT_EPS

int gdn_oracle_mutant_id(void) { return ORACLE_MUTANT; }
