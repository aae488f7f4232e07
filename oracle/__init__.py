"""CPU oracle for mask-driven block-sparse video attention (test infrastructure).

This package is the plain, slow, fp64 statement of what the GPU path must compute.
It is TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import it.  It shares no code with the HIP library and
imports nothing from it; the product path never calls into it.

Contents
  coords     token coordinates of an executed position (frame-, tile-, position-major,
             tile-major over a grid padded to whole tiles)
  masks      the boolean keep-predicate of each mask kind
  classify   per-(query-tile, key-tile) full / boundary / empty classes and lists
  attention  masked softmax attention written from its definition
  profile    the sampled-query head profiler and router
  reorder    the token permutations of the executed orders and their inverses
  merge      merging partial results over disjoint key sets by their log-sum-exp

Every function is pinned by tests under ``tests/`` (marked ``not gpu``) against
numbers the pages print, closed forms, special cases and brute force on tiny
inputs.  No function here is "parity unpinned".
"""
from .coords import token_coords, num_tiles, seq_len, padded_dims, is_real  # noqa: F401
from .masks import keep_matrix  # noqa: F401
from .classify import classify, EMPTY, FULL, BOUNDARY  # noqa: F401
from .classify import rounded_keep_rows  # noqa: F401
from .attention import attention  # noqa: F401
from .profile import profile_heads  # noqa: F401
from .reorder import layout_permutation, tile_major_permutation, reorder_tokens  # noqa: F401
from .merge import merge_partials  # noqa: F401
