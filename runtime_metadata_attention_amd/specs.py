"""MaskSpecs of the mask families measured for CompileMask.

Each spec has a forward section (Regions of query rows i; rules over keys j)
and a backward section (Regions of key columns j; rules over query rows i), as
the forward and backward passes use separate rules aligned with their
traversal (CompileMask paper summary, section 3.3).  The families follow the
evaluation's masks (section 4.1): causal, HSTU history/target, the
shared-prompt reward model (the "Region C" rule [0,b) u [s(i),i+1) of section
3.2.2) and a CLEAR-like multi-interval retrieval mask.
"""

CAUSAL = """
mask causal
forward
  region all: true => j <= i
backward
  region all: true => i >= j
"""

# prompt rows are causal; a response row sees the prompt and its own response
SHARED_PROMPT = """
mask shared_prompt
param P
forward
  region prompt:   i < P  => j <= i
  region response: i >= P => j < P | j in [start(seg(i)), i + 1)
backward
  region prompt:   j < P  => i >= j
  region response: j >= P => i in [j, end(seg(j)))
"""

# history rows are causal; a target row sees the whole history and itself
HSTU = """
mask hstu
param h
forward
  region history: i < h  => j <= i
  region target:  i >= h => j < h | j == i
backward
  region history: j < h  => i >= j
  region target:  j >= h => i == j
"""

# prefix rows are causal; a segment row sees the prefix, its own segment up to
# itself and the two segments it references; a segment key is seen by its own
# segment's later rows and by every segment that references its segment
RETRIEVAL = """
mask retrieval4
param g
refs 2
forward
  region prefix:  i < g  => j <= i
  region segment: i >= g => j < g | j in [start(seg(i)), i + 1) | j in ref(seg(i), 0) | j in ref(seg(i), 1)
backward
  region prefix:  j < g  => i >= j
  region segment: j >= g => i in [j, end(seg(j))) | exists k ((ref(k, 0) == seg(j) | ref(k, 1) == seg(j)) & i in k)
"""

BY_MASK = {
    "causal": CAUSAL,
    "shared_prompt": SHARED_PROMPT,
    "hstu": HSTU,
    "retrieval": RETRIEVAL,
}
