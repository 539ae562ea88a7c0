"""MI355X (gfx950) Domino draft-block rollout.

The rollout runs in hand-written HIP kernels behind a C ABI
(``libdomino_rollout.so``); ``rollout`` holds the thin ctypes binding and
``synth`` the seeded synthetic inputs.
"""
